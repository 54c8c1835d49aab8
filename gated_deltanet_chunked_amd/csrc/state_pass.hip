// state_pass.hip -- the sequential inter-chunk state pass fused with the chunk output.
//
// The "open-jev-fast" README ("Phase 3", item 1) keeps the fp32 recurrent state in registers and
// passes only the state from chunk to chunk.  Here one workgroup owns one (sequence, v-head,
// 16-column slice of the 128 value columns): the state slice H[:, cols] (128 x 16 fp32) lives in
// MFMA accumulators, spread over 4 compute waves (wave w holds key rows 32w .. 32w+31), and the
// chunks of the sequence are walked in order.  Sequences, heads and slices run in parallel.
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
// Data movement (one producer wave + four compute waves per workgroup):
//   * The producer wave streams each chunk's K tile (XOR-swizzled rows), the v-head's record
//     (T' hi/lo, P, decays) and the V tile into a 3-deep LDS ring with global->LDS loads
//     (global_load_lds_dwordx4: 1 KiB contiguous per instruction, no VGPRs), two chunks ahead of
//     the compute waves, and pulls the Q rows of the chunk after that into L2.
//   * The compute waves read every operand from LDS (K^T fragments come from the same K tile
//     through transposing LDS reads), except Q, which they load into registers one chunk ahead.
//   * LDS also carries the three cross-wave exchanges per chunk: bf16 H, R and U~.
#include "gdn_device.h"

namespace gdn {

namespace {

constexpr int kPitchH = kDim + 8;     // Ht row pitch (bf16): value column j, key index
constexpr int kPitchT = kChunk + 8;   // Rh/Rl/Uh/Ul/Uo row pitch (bf16): value column j, token
constexpr int kComputeWaves = 4;
constexpr int kThreads = 64 * (kComputeWaves + 1);
constexpr int kStages = 3;
// One ring stage: K tile (64 x 128 bf16, swizzled) | the v-head record | V tile (64 x 16 bf16).
constexpr int kStK = 0;
constexpr int kStRec = kStK + kChunk * kDim * 2;         // 16384
constexpr int kStV = kStRec + kRecBytes;                  // 35328
constexpr int kStageBytes = kStV + kChunk * kDvTile * 2;  // 37376
constexpr int kDmaK = kChunk * kDim * 2 / 1024;           // 16 instructions of 1 KiB
constexpr int kDmaRec = (kRecBytes + 1023) / 1024;        // 19 (the last one half full)
constexpr int kDmaV = kChunk * kDvTile * 2 / 1024;        // 2
constexpr int kDmaPerChunk = kDmaK + kDmaRec + kDmaV;     // 37
constexpr int kTouchQ = 2;                                // L2 pulls of one chunk's Q rows
static_assert(kStageBytes % 16 == 0 && kStRec % 16 == 0 && kStV % 16 == 0, "16-byte LDS slots");

// Byte offset of bf16 element (row, col) in a swizzled 64 x 128 tile: 16-byte chunks are
// XOR-permuted by row so that 16 lanes reading one chunk column of 16 rows hit distinct banks.
__device__ __forceinline__ int swz(int row, int col) {
  return row * (kDim * 2) + ((((col >> 3) ^ (row & 15))) << 4) + ((col & 7) << 1);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane (M0 holds the wave's
// LDS base).  Completion is tracked by this wave's vmcnt only.
__device__ __forceinline__ void dma16(const void *src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src) : "memory");
}
// 4 bytes per lane into a scratch LDS word: pulls the 128-byte line holding src into L2.
__device__ __forceinline__ void touch(const void *src, unsigned lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(src) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// hi = bf16(x), lo = bf16(x - hi) for two values at once (packed bf16 pairs).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
__device__ __forceinline__ void store_u32x2(unsigned short *dst, uint32_t a, uint32_t b) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2 *>(dst) = u32x2{a, b};
}
__device__ __forceinline__ bf16x8 lds_bf16x8(const void *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
// Transposing LDS read of 4 bf16 per lane (gfx950 ds_read_b64_tr_b16); p is 8-byte aligned LDS.
__device__ __forceinline__ v4i16 lds_read_tr16(const void *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
}

// Producer: one chunk's K tile, record and V tile into a ring stage (kDmaPerChunk instructions,
// issued unconditionally so the vmcnt bookkeeping is static; rows past the sequence end are
// clamped to its last row, which the compute waves never use).
__device__ __forceinline__ void dma_chunk(int c, int tb, int te, int slot0, int hk, int h, int Hk,
                                          int Hv, int d0, int l, const unsigned short *k,
                                          const unsigned short *v, const uint8_t *rec,
                                          unsigned stage_lds) {
  const int t0 = tb + kChunk * c;
  const int Lm1 = min(kChunk, te - t0) - 1;
#pragma unroll
  for (int m = 0; m < kDmaK; ++m) {
    const int row = 4 * m + (l >> 4);
    const int lc = (l & 15) ^ (row & 15);  // logical 16-byte chunk stored at physical chunk l & 15
    dma16(k + ((size_t)(t0 + min(row, Lm1)) * Hk + hk) * kDim + lc * 8, stage_lds + kStK + m * 1024);
  }
  const uint8_t *rp = rec + ((size_t)(slot0 + c) * Hv + h) * kRecBytes + l * 16;
#pragma unroll
  for (int m = 0; m < kDmaRec - 1; ++m) dma16(rp + m * 1024, stage_lds + kStRec + m * 1024);
  if (l < (kRecBytes - (kDmaRec - 1) * 1024) / 16)
    dma16(rp + (kDmaRec - 1) * 1024, stage_lds + kStRec + (kDmaRec - 1) * 1024);
#pragma unroll
  for (int m = 0; m < kDmaV; ++m) {
    const int row = 32 * m + (l >> 1);
    dma16(v + ((size_t)(t0 + min(row, Lm1)) * Hv + h) * kDim + d0 + 8 * (l & 1),
          stage_lds + kStV + m * 1024);
  }
}

__device__ __forceinline__ void touch_q(int c, int tb, int te, int hk, int Hk, int l,
                                        const unsigned short *q, unsigned sink) {
  const int t0 = tb + kChunk * c;
  const unsigned short *qr = q + ((size_t)(t0 + min(l, min(kChunk, te - t0) - 1)) * Hk + hk) * kDim;
  touch(qr, sink);
  touch(qr + 64, sink);
}

// Compute waves: Q rows 16w + (l%16) (clamped) as the A operands of Q H, one chunk ahead.
__device__ __forceinline__ void load_q(bf16x8 (&qx)[4], int c, int tb, int te, int hk, int Hk, int w,
                                       int l, const unsigned short *__restrict__ q) {
  const int t0 = tb + kChunk * c;
  const int row = min(16 * w + (l & 15), min(kChunk, te - t0) - 1);
  const unsigned short *qr = q + ((size_t)(t0 + row) * Hk + hk) * kDim + 8 * (l >> 4);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qx[ks] = load_bf16x8(qr + 32 * ks);
}

// One chunk on the compute waves.  Rows past the sequence end hold clamped data; they need no
// masking because T' has zero rows and columns there (beta = 0), so U~ is zero on them, and
// their output rows are never stored.
__device__ __forceinline__ void chunk_step(const unsigned char *st, const bf16x8 (&qx)[4], int t0,
                                           int te, int h, int Hv, int d0, int w, int l,
                                           f32x4 (&H)[2], unsigned short *Ht, unsigned short *Rh,
                                           unsigned short *Rl, unsigned short *Uh,
                                           unsigned short *Ul, unsigned short *Uo,
                                           unsigned short *__restrict__ o) {
  const int lj = l & 15, lg = l >> 4;
  const int L = min(kChunk, te - t0);
  const unsigned char *rs = st + kStRec;

  // K^T fragments for the state update, read transposed from the K tile: fragment (key block
  // 2w + a, token step ks), lane (lj, lg) holds K[token 32 ks + 8 lg + e][key 32 w + 16 a + lj].
  // ds_read_b64_tr_b16: within each 16-lane group, lane r names 4 consecutive bf16 (row r of a
  // 16 x 4 matrix M) and lane i receives M[4 j + i / 4][i % 4], j = 0..3.  With lane r = 4 j + q
  // naming K[token t + j][key base + 4 q .. + 3], lane i receives K[t .. t + 3][base + i]: half a
  // fragment (4 tokens) per read.
  bf16x8 kc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int key = 32 * w + 16 * a + 4 * (lj & 3);
      const int tok = 32 * ks + 8 * lg + (lj >> 2);
      const v4i16 lo4 = lds_read_tr16(st + kStK + swz(tok, key));
      const v4i16 hi4 = lds_read_tr16(st + kStK + swz(tok + 4, key));
      kc[a][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }

  // X = K H and Q H (contraction over the 128 keys; B operand = bf16 H from LDS)
  f32x4 X = zero4(), O = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 hb = lds_bf16x8(&Ht[lj * kPitchH + 32 * ks + 8 * lg]);
    const bf16x8 kx = lds_bf16x8(st + kStK + swz(16 * w + lj, 32 * ks + 8 * lg));
    X = mfma_bf16(kx, hb, X);
    O = mfma_bf16(qx[ks], hb, O);
  }
  const f32x4 eg = *reinterpret_cast<const f32x4 *>(rs + kRecEG + (16 * w + 4 * lg) * 4);
  const f32x4 ed = *reinterpret_cast<const f32x4 *>(rs + kRecED + (16 * w + 4 * lg) * 4);
  const float egc = *reinterpret_cast<const float *>(rs + kRecEG + 63 * 4);
  float vv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
    vv[rr] = bits_to_float(*reinterpret_cast<const unsigned short *>(
        st + kStV + ((16 * w + 4 * lg + rr) * kDvTile + lj) * 2));

  // R = V - e^G o X (hi/lo to LDS, value-major); O <- e^G o O
  {
    float R[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      R[rr] = vv[rr] - eg[rr] * X[rr];
      O[rr] *= eg[rr];
    }
    uint32_t h0, l0, h1, l1;
    split_pair(R[0], R[1], h0, l0);
    split_pair(R[2], R[3], h1, l1);
    store_u32x2(&Rh[lj * kPitchT + 16 * w + 4 * lg], h0, h1);
    store_u32x2(&Rl[lj * kPitchT + 16 * w + 4 * lg], l0, l1);
  }
  __syncthreads();

  // U~ = T' R for row block w (3 hi/lo terms; row blocks 2, 3 need two token steps)
  const int fb = w < 2 ? w : 2 * w - 2;
  f32x4 U = zero4();
  {
    const bf16x8 th = lds_bf16x8(rs + kRecTpHi + fb * kFragBytes + l * 16);
    const bf16x8 tl = lds_bf16x8(rs + kRecTpLo + fb * kFragBytes + l * 16);
    const bf16x8 bh = lds_bf16x8(&Rh[lj * kPitchT + 8 * lg]);
    const bf16x8 bl = lds_bf16x8(&Rl[lj * kPitchT + 8 * lg]);
    U = mfma_bf16(th, bh, U);
    U = mfma_bf16(th, bl, U);
    U = mfma_bf16(tl, bh, U);
    if (w >= 2) {
      const bf16x8 th1 = lds_bf16x8(rs + kRecTpHi + (fb + 1) * kFragBytes + l * 16);
      const bf16x8 tl1 = lds_bf16x8(rs + kRecTpLo + (fb + 1) * kFragBytes + l * 16);
      const bf16x8 bh1 = lds_bf16x8(&Rh[lj * kPitchT + 32 + 8 * lg]);
      const bf16x8 bl1 = lds_bf16x8(&Rl[lj * kPitchT + 32 + 8 * lg]);
      U = mfma_bf16(th1, bh1, U);
      U = mfma_bf16(th1, bl1, U);
      U = mfma_bf16(tl1, bh1, U);
    }
  }
  {
    uint32_t h0, l0, h1, l1;
    split_pair(ed[0] * U[0], ed[1] * U[1], h0, l0);
    split_pair(ed[2] * U[2], ed[3] * U[3], h1, l1);
    store_u32x2(&Uh[lj * kPitchT + 16 * w + 4 * lg], h0, h1);
    store_u32x2(&Ul[lj * kPitchT + 16 * w + 4 * lg], l0, l1);
    store_u32x2(&Uo[lj * kPitchT + 16 * w + 4 * lg], pack_bf16x2(U[0], U[1]),
                pack_bf16x2(U[2], U[3]));
  }
  __syncthreads();

  // o = e^G o (Q H) + P U~
  {
    O = mfma_bf16(lds_bf16x8(rs + kRecP + fb * kFragBytes + l * 16),
                  lds_bf16x8(&Uo[lj * kPitchT + 8 * lg]), O);
    if (w >= 2)
      O = mfma_bf16(lds_bf16x8(rs + kRecP + (fb + 1) * kFragBytes + l * 16),
                    lds_bf16x8(&Uo[lj * kPitchT + 32 + 8 * lg]), O);
    const uint32_t p01 = pack_bf16x2(O[0], O[1]), p23 = pack_bf16x2(O[2], O[3]);
    const unsigned short ob[4] = {(unsigned short)p01, (unsigned short)(p01 >> 16),
                                  (unsigned short)p23, (unsigned short)(p23 >> 16)};
    unsigned short *orow = o + ((size_t)(t0 + 16 * w + 4 * lg) * Hv + h) * kDim + d0 + lj;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (16 * w + 4 * lg + rr < L) orow[(size_t)rr * Hv * kDim] = ob[rr];
  }

  // H = e^{G_last} H + K^T (e^{G_last - G} o U~)  (decayed U~ hi + lo)
#pragma unroll
  for (int a = 0; a < 2; ++a) H[a] *= egc;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8 bh = lds_bf16x8(&Uh[lj * kPitchT + 32 * ks + 8 * lg]);
    const bf16x8 bl = lds_bf16x8(&Ul[lj * kPitchT + 32 * ks + 8 * lg]);
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      H[a] = mfma_bf16(kc[a][ks], bh, H[a]);
      H[a] = mfma_bf16(kc[a][ks], bl, H[a]);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
    store_u32x2(&Ht[lj * kPitchH + 32 * w + 16 * a + 4 * lg], pack_bf16x2(H[a][0], H[a][1]),
                pack_bf16x2(H[a][2], H[a][3]));
  __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void state_pass_kernel(
    const unsigned short *__restrict__ q, const unsigned short *__restrict__ k,
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const float *h0, unsigned short *__restrict__ o, float *hT,  // hT may equal h0
    const uint8_t *__restrict__ rec, int Hk, int Hv) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[kStages * kStageBytes];
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
    // Producer wave.  Barriers: one before the loop, three per chunk, as the compute waves.
    if (nc > 0) {
      const unsigned ring_lds = (unsigned)(uintptr_t)ring;
      const unsigned sink = (unsigned)(uintptr_t)touch_sink;
      const bool lead = tile == 0 && (h % (Hv / Hk)) == 0;  // one Q-warming workgroup per k-head
      if (lead)
        for (int c = 0; c < 3; ++c) touch_q(min(c, nc - 1), tb, te, hk, Hk, l, q, sink);
      dma_chunk(0, tb, te, slot0, hk, h, Hk, Hv, d0, l, k, v, rec, ring_lds);
      dma_chunk(min(1, nc - 1), tb, te, slot0, hk, h, Hk, Hv, d0, l, k, v, rec,
                ring_lds + kStageBytes);
      wait_vmcnt<kDmaPerChunk>();  // chunk 0 has landed
      __syncthreads();
      for (int c = 0; c < nc; ++c) {
        // Stage (c + 2) % 3 held chunk c - 1, which every compute wave finished before the last
        // barrier; the clamped reload of the last chunk is never read.
        if (lead) touch_q(min(c + 3, nc - 1), tb, te, hk, Hk, l, q, sink);
        dma_chunk(min(c + 2, nc - 1), tb, te, slot0, hk, h, Hk, Hv, d0, l, k, v, rec,
                  ring_lds + ((c + 2) % kStages) * kStageBytes);
        __syncthreads();
        __syncthreads();
        // Chunk c + 1 must have landed before the end-of-chunk barrier: only this iteration's
        // loads may still be in flight.
        if (lead) wait_vmcnt<kDmaPerChunk + kTouchQ>(); else wait_vmcnt<kDmaPerChunk>();
        __syncthreads();
      }
    }
    wait_vmcnt<0>();  // no LDS write may land after the workgroup ends
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
    for (int a = 0; a < 2; ++a)
      store_u32x2(&Ht[lj * kPitchH + 32 * w + 16 * a + 4 * lg], pack_bf16x2(H[a][0], H[a][1]),
                  pack_bf16x2(H[a][2], H[a][3]));
    bf16x8 qa[4], qb[4];
    load_q(qa, 0, tb, te, hk, Hk, w, l, q);
    __syncthreads();
    for (int c = 0; c < nc; c += 2) {
      load_q(qb, min(c + 1, nc - 1), tb, te, hk, Hk, w, l, q);
      chunk_step(ring + (c % kStages) * kStageBytes, qa, tb + kChunk * c, te, h, Hv, d0, w, l, H,
                 Ht, Rh, Rl, Uh, Ul, Uo, o);
      if (c + 1 < nc) {
        load_q(qa, min(c + 2, nc - 1), tb, te, hk, Hk, w, l, q);
        chunk_step(ring + ((c + 1) % kStages) * kStageBytes, qb, tb + kChunk * (c + 1), te, h, Hv,
                   d0, w, l, H, Ht, Rh, Rl, Uh, Ul, Uo, o);
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
                       const float *h0, void *o, float *hT, const void *rec, int N, int Hk, int Hv,
                       hipStream_t stream) {
  const unsigned nblocks = (unsigned)N * (unsigned)Hv * kDvTiles;
  hipLaunchKernelGGL(state_pass_kernel, dim3(nblocks), dim3(kThreads), 0, stream,
                     static_cast<const unsigned short *>(q), static_cast<const unsigned short *>(k),
                     static_cast<const unsigned short *>(v), cu, h0,
                     static_cast<unsigned short *>(o), hT, static_cast<const uint8_t *>(rec), Hk, Hv);
}

}  // namespace gdn
