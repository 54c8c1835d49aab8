// state_pass.hip -- the sequential inter-chunk state pass fused with the chunk output.
//
// The "open-jev-fast" README ("Phase 3", item 1) keeps the fp32 recurrent state in registers and
// passes only the state from chunk to chunk.  Here one workgroup owns one (sequence, v-head,
// 16-column slice of the 128 value columns): the state slice H[:, cols] (128 x 16 fp32) lives in
// MFMA accumulators, spread over 4 waves (wave w holds key rows 32w .. 32w+31), and the chunks
// of the sequence are walked in order.  Sequences, heads and slices run in parallel.
//
// With H = S^T (key-major), local cumsum G, T' = (I + A)^-1 diag(beta) and
// P = tril(Q K^T o e^{G_i - G_j}) from chunk_prep.hip, one chunk is
//     X  = K H                                   (bf16 K x bf16 H, fp32 accumulate)
//     R  = V - e^{G} o X
//     U~ = T' R                                  (T' and R split hi/lo: 3 MFMA terms)
//     o  = e^{G} o (Q H) + P U~                  (output path in plain bf16)
//     H  = e^{G_last} H + K^T (e^{G_last - G} o U~)   (decayed U~ split hi/lo: 2 MFMA terms)
// which is the chunked form of the gated delta rule: (I + A) U~ = diag(beta)(V - e^G o K H).
// The hi/lo splits keep the state path at about 16 significant bits per operand, so the fp32
// state does not drift over hundreds of chunks; bf16 is used where only the output sees it.
//
// Operands reach registers straight from global memory (one chunk ahead, double-buffered in
// registers); LDS only carries the three cross-wave exchanges per chunk: bf16 H, R and U~.
// A fifth wave hides HBM latency: it runs kTouchAhead chunks ahead and pulls every line the
// compute waves will load into L2, so their one-chunk-ahead register prefetch hits in L2.
#include "gdn_device.h"

namespace gdn {

namespace {

constexpr int kPitchH = kDim + 8;     // Ht row pitch (bf16): value column j, key index
constexpr int kPitchT = kChunk + 8;   // Rh/Rl/Uh/Ul/Uo row pitch (bf16): value column j, token
constexpr int kComputeWaves = 4;
constexpr int kThreads = 64 * (kComputeWaves + 1);  // + one L2-warming wave
constexpr int kTouchAhead = 4;        // chunks the warming wave runs ahead of the compute waves

// One 4-byte load per lane, delivered straight into a scratch LDS word (global_load_lds_dword):
// it pulls the 128-byte line into L2 without occupying a VGPR, so the warming wave never has to
// wait for it.  Lane i writes LDS byte lds_dummy + 4 i.
__device__ __forceinline__ void touch(const void *p, unsigned lds_dummy) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_dummy), "v"(p)
               : "memory");
}

// Bring chunk c's operands into L2: the lead workgroup of each sharing group touches the data it
// shares (K, Q and K^T of the k-head; the v-head's record), every workgroup touches its V slice.
__device__ __forceinline__ void touch_chunk(int c, int tb, int te, int slot0, int hk, int h, int Hk,
                                            int Hv, int d0, bool lead_k, bool lead_v, int l,
                                            const unsigned short *q, const unsigned short *k,
                                            const unsigned short *v, const uint8_t *rec,
                                            const uint8_t *kcrec, unsigned lds_dummy) {
  const int t0 = tb + kChunk * c;
  const int L = min(kChunk, te - t0);
  const int row = min(l, L - 1);
  const size_t slot = (size_t)slot0 + c;
  if (lead_k) {
    const unsigned short *kr = k + ((size_t)(t0 + row) * Hk + hk) * kDim;
    const unsigned short *qr = q + ((size_t)(t0 + row) * Hk + hk) * kDim;
    touch(kr, lds_dummy);
    touch(kr + 64, lds_dummy);
    touch(qr, lds_dummy);
    touch(qr + 64, lds_dummy);
    const uint8_t *kc = kcrec + (slot * Hk + hk) * kKcBytes + l * 128;
    touch(kc, lds_dummy);
    touch(kc + 8192, lds_dummy);
  }
  if (lead_v) {
    const uint8_t *rp = rec + (slot * Hv + h) * kRecBytes;
    touch(rp + l * 128, lds_dummy);
    touch(rp + 8192 + l * 128, lds_dummy);
    touch(rp + 16384 + min(l, (kRecBytes - 16384) / 128 - 1) * 128, lds_dummy);
  }
  touch(v + ((size_t)(t0 + row) * Hv + h) * kDim + d0, lds_dummy);
}

// Operands of one chunk, exactly as loaded: nothing here is touched until the chunk is
// processed, so the loads stay in flight while the previous chunk computes.
struct ChunkOps {
  bf16x8 kx[4];      // K rows 16w + (l%16) (clamped), all 128 keys: A operands of X = K H
  bf16x8 qx[4];      // Q rows, A operands of Q H
  bf16x8 kc[2][2];   // K^T fragments (key block 2w + a, token step ks)
  bf16x8 tph[2], tpl[2], pf[2];  // T' hi, T' lo, P fragments of row block w
  unsigned short vb[4];  // V[token 16w + 4(l/16) + r][col l%16] (clamped), raw bf16
  f32x4 eg, ed;      // e^{G}, e^{G_last - G} for the same 4 tokens
  float egc;         // e^{G_last}
};

__device__ __forceinline__ void load_chunk(ChunkOps &op, int c, int tb, int te, int slot0, int hk,
                                           int h, int Hk, int Hv, int d0, int w, int l,
                                           const unsigned short *__restrict__ q,
                                           const unsigned short *__restrict__ k,
                                           const unsigned short *__restrict__ v,
                                           const uint8_t *__restrict__ rec,
                                           const uint8_t *__restrict__ kcrec) {
  const int lj = l & 15, lg = l >> 4;
  const int t0 = tb + kChunk * c;
  const int L = min(kChunk, te - t0);
  const size_t slot = (size_t)slot0 + c;
  // Every load is unconditional, with rows past the end clamped to the last row: a load under a
  // divergent branch would make the compiler drain all outstanding loads right after it,
  // including the prefetch of the next chunk.  The clamped rows need no masking: T' has zero
  // rows and columns there (beta = 0), so U~ is zero on them whatever X and V hold, and their
  // output rows are never stored.
  const int row = 16 * w + lj;
  const size_t base = ((size_t)(t0 + min(row, L - 1)) * Hk + hk) * kDim + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    op.kx[ks] = load_bf16x8(k + base + 32 * ks);
    op.qx[ks] = load_bf16x8(q + base + 32 * ks);
  }
  const uint8_t *kcp = kcrec + (slot * Hk + hk) * kKcBytes + l * 16;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) op.kc[a][ks] = load_bf16x8(kcp + ((2 * w + a) * 2 + ks) * kFragBytes);
  const uint8_t *rp = rec + (slot * Hv + h) * kRecBytes;
  const int fb = w < 2 ? w : 2 * w - 2;
  op.tph[0] = load_bf16x8(rp + kRecTpHi + fb * kFragBytes + l * 16);
  op.tpl[0] = load_bf16x8(rp + kRecTpLo + fb * kFragBytes + l * 16);
  op.pf[0] = load_bf16x8(rp + kRecP + fb * kFragBytes + l * 16);
  if (w >= 2) {
    op.tph[1] = load_bf16x8(rp + kRecTpHi + (fb + 1) * kFragBytes + l * 16);
    op.tpl[1] = load_bf16x8(rp + kRecTpLo + (fb + 1) * kFragBytes + l * 16);
    op.pf[1] = load_bf16x8(rp + kRecP + (fb + 1) * kFragBytes + l * 16);
  } else {
    op.tph[1] = op.tpl[1] = op.pf[1] = zero_bf16x8();
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int tr = 16 * w + 4 * lg + rr;
    op.vb[rr] = v[((size_t)(t0 + min(tr, L - 1)) * Hv + h) * kDim + d0 + lj];
  }
  op.eg = *reinterpret_cast<const f32x4 *>(rp + kRecEG + (16 * w + 4 * lg) * 4);
  op.ed = *reinterpret_cast<const f32x4 *>(rp + kRecED + (16 * w + 4 * lg) * 4);
  op.egc = *reinterpret_cast<const float *>(rp + kRecEG + 63 * 4);
}

__device__ __forceinline__ void write_pair4(unsigned short *dst, const __bf16 *x) {
  // four consecutive bf16 (8 bytes, 8-byte aligned)
  const uint32_t lo = (uint32_t)bf16_bits(x[0]) | ((uint32_t)bf16_bits(x[1]) << 16);
  const uint32_t hi = (uint32_t)bf16_bits(x[2]) | ((uint32_t)bf16_bits(x[3]) << 16);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2 *>(dst) = u32x2{lo, hi};
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const unsigned short *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// One chunk: X = K H, R, U~ = T' R, output, state update.  Three workgroup barriers.
__device__ __forceinline__ void chunk_step(const ChunkOps &cur, int t0, int te, int h, int Hv,
                                           int d0, int w, int l, f32x4 (&H)[2],
                                           unsigned short *Ht, unsigned short *Rh,
                                           unsigned short *Rl, unsigned short *Uh,
                                           unsigned short *Ul, unsigned short *Uo,
                                           unsigned short *__restrict__ o) {
  const int lj = l & 15, lg = l >> 4;
  const int L = min(kChunk, te - t0);

  // X = K H and Q H (contraction over the 128 keys; B operand = bf16 H from LDS)
  f32x4 X = zero4(), O = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 hb = lds_bf16x8(&Ht[lj * kPitchH + 32 * ks + 8 * lg]);
    X = mfma_bf16(cur.kx[ks], hb, X);
    O = mfma_bf16(cur.qx[ks], hb, O);
  }
  // R = V - e^G o X (hi/lo to LDS, value-major); O <- e^G o O
  {
    __bf16 rh[4], rl[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      split_hilo(bits_to_float(cur.vb[rr]) - cur.eg[rr] * X[rr], rh[rr], rl[rr]);
      O[rr] *= cur.eg[rr];
    }
    write_pair4(&Rh[lj * kPitchT + 16 * w + 4 * lg], rh);
    write_pair4(&Rl[lj * kPitchT + 16 * w + 4 * lg], rl);
  }
  __syncthreads();

  // U~ = T' R for row block w (3 hi/lo terms; row blocks 2, 3 need two token steps)
  f32x4 U = zero4();
  {
    const bf16x8 bh = lds_bf16x8(&Rh[lj * kPitchT + 8 * lg]);
    const bf16x8 bl = lds_bf16x8(&Rl[lj * kPitchT + 8 * lg]);
    U = mfma_bf16(cur.tph[0], bh, U);
    U = mfma_bf16(cur.tph[0], bl, U);
    U = mfma_bf16(cur.tpl[0], bh, U);
    if (w >= 2) {
      const bf16x8 bh1 = lds_bf16x8(&Rh[lj * kPitchT + 32 + 8 * lg]);
      const bf16x8 bl1 = lds_bf16x8(&Rl[lj * kPitchT + 32 + 8 * lg]);
      U = mfma_bf16(cur.tph[1], bh1, U);
      U = mfma_bf16(cur.tph[1], bl1, U);
      U = mfma_bf16(cur.tpl[1], bh1, U);
    }
  }
  {
    __bf16 uh[4], ul[4], uo[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      split_hilo(cur.ed[rr] * U[rr], uh[rr], ul[rr]);
      uo[rr] = to_bf16(U[rr]);
    }
    write_pair4(&Uh[lj * kPitchT + 16 * w + 4 * lg], uh);
    write_pair4(&Ul[lj * kPitchT + 16 * w + 4 * lg], ul);
    write_pair4(&Uo[lj * kPitchT + 16 * w + 4 * lg], uo);
  }
  __syncthreads();

  // o = e^G o (Q H) + P U~
  {
    const bf16x8 b0 = lds_bf16x8(&Uo[lj * kPitchT + 8 * lg]);
    O = mfma_bf16(cur.pf[0], b0, O);
    if (w >= 2) {
      const bf16x8 b1 = lds_bf16x8(&Uo[lj * kPitchT + 32 + 8 * lg]);
      O = mfma_bf16(cur.pf[1], b1, O);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int tr = 16 * w + 4 * lg + rr;
      if (tr < L) o[((size_t)(t0 + tr) * Hv + h) * kDim + d0 + lj] = bf16_bits(to_bf16(O[rr]));
    }
  }

  // H = e^{G_last} H + K^T (e^{G_last - G} o U~)  (decayed U~ hi + lo)
#pragma unroll
  for (int a = 0; a < 2; ++a) H[a] *= cur.egc;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 bh = lds_bf16x8(&Uh[lj * kPitchT + 32 * ks + 8 * lg]);
    const bf16x8 bl = lds_bf16x8(&Ul[lj * kPitchT + 32 * ks + 8 * lg]);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      H[a] = mfma_bf16(cur.kc[a][ks], bh, H[a]);
      H[a] = mfma_bf16(cur.kc[a][ks], bl, H[a]);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    __bf16 hb[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) hb[rr] = to_bf16(H[a][rr]);
    write_pair4(&Ht[lj * kPitchH + 32 * w + 16 * a + 4 * lg], hb);
  }
  __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void state_pass_kernel(
    const unsigned short *__restrict__ q, const unsigned short *__restrict__ k,
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const float *h0, unsigned short *__restrict__ o, float *hT,  // hT may equal h0
    const uint8_t *__restrict__ rec, const uint8_t *__restrict__ kcrec, int Hk, int Hv) {
  __shared__ __attribute__((aligned(16))) unsigned short Ht[kDvTile * kPitchH];
  __shared__ __attribute__((aligned(16))) unsigned short Rh[kDvTile * kPitchT];
  __shared__ __attribute__((aligned(16))) unsigned short Rl[kDvTile * kPitchT];
  __shared__ __attribute__((aligned(16))) unsigned short Uh[kDvTile * kPitchT];
  __shared__ __attribute__((aligned(16))) unsigned short Ul[kDvTile * kPitchT];
  __shared__ __attribute__((aligned(16))) unsigned short Uo[kDvTile * kPitchT];
  __shared__ __attribute__((aligned(16))) unsigned int touch_sink[64];

  const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tile = lid % kDvTiles;
  const int rest = lid / kDvTiles;
  const int h = rest % Hv, n = rest / Hv;
  const int hk = h / (Hv / Hk);
  const int d0 = kDvTile * tile;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lj = l & 15, lg = l >> 4;
  const int tb = cu[n], te = cu[n + 1];
  const int nc = (te - tb + kChunk - 1) / kChunk;
  const int slot0 = tb / kChunk + n;
  const size_t state_base = ((size_t)n * Hv + h) * kDim * kDim;

  if (w == kComputeWaves) {
    // L2-warming wave: stays kTouchAhead chunks ahead, joining the compute waves' barriers (one
    // before the loop, three per chunk) so it neither lags nor runs away.
    const unsigned sink = (unsigned)(uintptr_t)touch_sink;
    const bool lead_v = tile == 0, lead_k = lead_v && (h % (Hv / Hk)) == 0;
    if (nc > 0) {
      for (int c = 0; c < min(kTouchAhead, nc); ++c)
        touch_chunk(c, tb, te, slot0, hk, h, Hk, Hv, d0, lead_k, lead_v, l, q, k, v, rec, kcrec, sink);
      __syncthreads();
      for (int c = 0; c < nc; ++c) {
        if (c + kTouchAhead < nc)
          touch_chunk(c + kTouchAhead, tb, te, slot0, hk, h, Hk, Hv, d0, lead_k, lead_v, l, q, k, v, rec,
                      kcrec, sink);
        __syncthreads();
        __syncthreads();
        __syncthreads();
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS write may land after the workgroup ends
    return;
  }

  // State slice: H[a][rr] = H[key 32w + 16a + 4 lg + rr][value d0 + lj].
  f32x4 H[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = 32 * w + 16 * a + 4 * lg + rr;
      H[a][rr] = h0 ? h0[state_base + (size_t)key * kDim + d0 + lj] : 0.f;
    }

  if (nc > 0) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      __bf16 hb[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) hb[rr] = to_bf16(H[a][rr]);
      write_pair4(&Ht[lj * kPitchH + 32 * w + 16 * a + 4 * lg], hb);
    }
    __syncthreads();

    // Ping-pong between two operand sets: chunk c + 1 loads while chunk c computes.
    ChunkOps A, B;
    load_chunk(A, 0, tb, te, slot0, hk, h, Hk, Hv, d0, w, l, q, k, v, rec, kcrec);
    for (int c = 0; c < nc; c += 2) {
      load_chunk(B, min(c + 1, nc - 1), tb, te, slot0, hk, h, Hk, Hv, d0, w, l, q, k, v, rec, kcrec);
      chunk_step(A, tb + kChunk * c, te, h, Hv, d0, w, l, H, Ht, Rh, Rl, Uh, Ul, Uo, o);
      if (c + 1 < nc) {
        load_chunk(A, min(c + 2, nc - 1), tb, te, slot0, hk, h, Hk, Hv, d0, w, l, q, k, v, rec, kcrec);
        chunk_step(B, tb + kChunk * (c + 1), te, h, Hv, d0, w, l, H, Ht, Rh, Rl, Uh, Ul, Uo, o);
      }
    }
  }

  if (hT) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 32 * w + 16 * a + 4 * lg + rr;
        hT[state_base + (size_t)key * kDim + d0 + lj] = H[a][rr];
      }
  }
}

void launch_state_pass(const void *q, const void *k, const void *v, const int32_t *cu,
                       const float *h0, void *o, float *hT, const void *rec, const void *kcrec,
                       int N, int Hk, int Hv, hipStream_t stream) {
  const unsigned nblocks = (unsigned)N * (unsigned)Hv * kDvTiles;
  hipLaunchKernelGGL(state_pass_kernel, dim3(nblocks), dim3(kThreads), 0, stream,
                     static_cast<const unsigned short *>(q), static_cast<const unsigned short *>(k),
                     static_cast<const unsigned short *>(v), cu, h0,
                     static_cast<unsigned short *>(o), hT, static_cast<const uint8_t *>(rec),
                     static_cast<const uint8_t *>(kcrec), Hk, Hv);
}

}  // namespace gdn
