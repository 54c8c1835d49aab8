// chunk_prep.hip -- state-independent work of every 64-token chunk, all chunks in parallel.
//
// The "open-jev-fast" README ("Phase 3", item 1) lists the steps of a chunk: gate cumsum,
// K K^T, the (I + A)^-1 solve, u and w, the chunk output and the state update; it also notes that
// the work which does not depend on the recurrent state can run for several chunks side by
// side while only the state is passed in sequence.  This kernel does all of that state-independent
// work for every (chunk, k-head) at once; the sequential part lives in state_pass.hip.
//
// Per (chunk, k-head) workgroup (4 waves):
//   1. K K^T and Q K^T (lower block triangle, 64 x 64) on bf16 MFMA with fp32 accumulation,
//      computed once and shared by the Hv/Hk value heads of the group.
//   2. K^T written out as MFMA A-operand fragments for the state pass.
//   3. per value head h of the group:
//        G   = inclusive cumsum of g inside the chunk (one wave64 scan, 64 tokens = 64 lanes)
//        A   = beta_i e^{G_i - G_j} (k_i . k_j) for i > j
//        T   = (I + A)^-1: diagonal 16x16 blocks by forward substitution, off-diagonal blocks
//              by the block recurrence T_ij = -T_ii sum_m A_im T_mj on fp32 MFMA
//        T'  = T diag(beta)                 -> bf16 hi + lo fragments (~16 significant bits)
//        P   = tril(Q K^T o e^{G_i - G_j})  -> bf16 fragments (output path only)
//        e^{G_i}, e^{G_last - G_i}          -> fp32
//      Every exponent is <= 0; e^{-G} is never formed.
// Tokens past the end of a sequence's last chunk enter as k = q = 0, g = 0, beta = 0, which
// leaves T' and P zero on those rows and columns.
#include "gdn_device.h"

namespace gdn {

namespace {

constexpr int kPitchF = 68;                       // fp32 row pitch of 64 x 64 LDS matrices
constexpr int kMatBytes = kChunk * kPitchF * 4;   // 17408
// LDS map: [Ks | Qs] (bf16, swizzled) share space with [As | Ts] (fp32); then Skk, Sqk, G, beta.
constexpr int kOffKs = 0;
constexpr int kOffQs = kChunk * kDim * 2;         // 16384
constexpr int kOffAs = 0;
constexpr int kOffTs = kMatBytes;
constexpr int kRegion0 = 2 * kMatBytes;           // >= 2 * 16384
constexpr int kOffSkk = kRegion0;
constexpr int kOffSqk = kOffSkk + kMatBytes;
constexpr int kOffG = kOffSqk + kMatBytes;
constexpr int kOffB = kOffG + kChunk * 4;
constexpr int kLdsBytes = kOffB + kChunk * 4;     // 70144

// Byte offset of bf16 element (row, col) in a swizzled 64 x 128 tile: 16-byte chunks are
// XOR-permuted by row so that 16 lanes reading one chunk column of 16 rows hit distinct banks.
__device__ __forceinline__ int swz(int row, int col) {
  return row * (kDim * 2) + ((((col >> 3) ^ (row & 15))) << 4) + ((col & 7) << 1);
}

}  // namespace

__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const unsigned short *__restrict__ q, const unsigned short *__restrict__ k,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int N, int Hk, int Hv, uint8_t *__restrict__ rec,
    uint8_t *__restrict__ kcrec) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
  unsigned char *Ks = smem + kOffKs;
  unsigned char *Qs = smem + kOffQs;
  float *As = reinterpret_cast<float *>(smem + kOffAs);
  float *Ts = reinterpret_cast<float *>(smem + kOffTs);
  float *Skk = reinterpret_cast<float *>(smem + kOffSkk);
  float *Sqk = reinterpret_cast<float *>(smem + kOffSqk);
  float *Gs = reinterpret_cast<float *>(smem + kOffG);
  float *Bs = reinterpret_cast<float *>(smem + kOffB);

  const int slot = blockIdx.x, hk = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lj = l & 15, lg = l >> 4;

  // Which (sequence, chunk) owns this slot: the largest n with cu[n]/64 + n <= slot.
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] / kChunk + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int n = lo;
  const int c = slot - (cu[n] / kChunk + n);
  const int t0 = cu[n] + kChunk * c, tend = cu[n + 1];
  if (t0 >= tend) return;  // slot unused (uniform across the workgroup)
  const int L = min(kChunk, tend - t0);
  const int r = Hv / Hk;

  // ---- 1. stage K and Q rows (zero past the sequence end) -------------------------------
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int p = tid + 256 * it, row = p >> 4, ch = p & 15;
    u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
    if (row < L) {
      const size_t off = ((size_t)(t0 + row) * Hk + hk) * kDim + ch * 8;
      kv = *reinterpret_cast<const u32x4 *>(k + off);
      qv = *reinterpret_cast<const u32x4 *>(q + off);
    }
    const int so = row * (kDim * 2) + ((ch ^ (row & 15)) << 4);
    *reinterpret_cast<u32x4 *>(Ks + so) = kv;
    *reinterpret_cast<u32x4 *>(Qs + so) = qv;
  }
  __syncthreads();

  // ---- 2. K K^T and Q K^T, lower 16x16 block triangle: 20 block products over 4 waves ----
#pragma unroll
  for (int it = 0; it < 5; ++it) {
    const int p = w + 4 * it;
    const int which = p >= 10 ? 1 : 0;
    const int b = p - 10 * which;
    const int rb = b < 1 ? 0 : (b < 3 ? 1 : (b < 6 ? 2 : 3));
    const int cb = b - rb * (rb + 1) / 2;
    const unsigned char *Am = which ? Qs : Ks;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 4 * ks + lg;
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Am + swz(16 * rb + lj, ch * 8));
      const bf16x8 bb = *reinterpret_cast<const bf16x8 *>(Ks + swz(16 * cb + lj, ch * 8));
      acc = mfma_bf16(a, bb, acc);
    }
    float *S = which ? Sqk : Skk;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) S[(16 * rb + 4 * lg + rr) * kPitchF + 16 * cb + lj] = acc[rr];
  }

  // ---- 3. K^T fragments for the state pass: fragment (rb, ks), lane ll holds
  //         K[token 32 ks + 8 (ll/16) + e][dk 16 rb + ll % 16], e = 0..7 ----------------
  {
    uint8_t *kcp = kcrec + ((size_t)slot * Hk + hk) * kKcBytes;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int s = tid + 256 * it, f = s >> 6, ll = s & 63;
      const int rb = f >> 1, ks = f & 1;
      const int dk = 16 * rb + (ll & 15);
      const int tok0 = 32 * ks + 8 * (ll >> 4);
      u16x8 vals;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vals[e] = *reinterpret_cast<const unsigned short *>(Ks + swz(tok0 + e, dk));
      *reinterpret_cast<u16x8 *>(kcp + f * kFragBytes + ll * 16) = vals;
    }
  }

  // ---- 4. per value head of this k-head group --------------------------------------------
  for (int jh = 0; jh < r; ++jh) {
    const int h = hk * r + jh;
    uint8_t *R = rec + ((size_t)slot * Hv + h) * kRecBytes;

    if (w == 0) {
      float gv = 0.f, bv = 0.f;
      if (l < L) {
        gv = g[(size_t)(t0 + l) * Hv + h];
        bv = beta[(size_t)(t0 + l) * Hv + h];
      }
      const float G = wave_inclusive_scan(gv);
      const float Glast = __shfl(G, 63, 64);
      Gs[l] = G;
      Bs[l] = bv;
      reinterpret_cast<float *>(R + kRecEG)[l] = expf(G);
      reinterpret_cast<float *>(R + kRecED)[l] = expf(Glast - G);
    }
    __syncthreads();

    // A = strictly lower beta_i e^{G_i - G_j} (k_i . k_j)
    for (int e = tid; e < kChunk * kChunk; e += 256) {
      const int i = e >> 6, j = e & 63;
      float a = 0.f;
      if (j < i) a = Bs[i] * expf(Gs[i] - Gs[j]) * Skk[i * kPitchF + j];
      As[i * kPitchF + j] = a;
    }
    __syncthreads();

    // Diagonal blocks: wave w inverts (I + A_ww) column by column (lanes 0..15 = columns).
    if (l < 16) {
      const int cj = l;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) s += As[(16 * w + i) * kPitchF + 16 * w + m] * x[m];
        x[i] = (i < cj) ? 0.f : (i == cj ? 1.f : -s);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(16 * w + i) * kPitchF + 16 * w + cj] = x[i];
    }
    __syncthreads();

    // Off-diagonal blocks, one sub-diagonal at a time: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
      if (w < 4 - d) {
        const int bi = w + d, bj = w;
        f32x4 S = zero4();
        for (int m = bj; m < bi; ++m) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const float a = As[(16 * bi + lj) * kPitchF + 16 * m + 4 * s4 + lg];
            const float bb = Ts[(16 * m + 4 * s4 + lg) * kPitchF + 16 * bj + lj];
            S = mfma_f32(a, bb, S);
          }
        }
        // S is fed back as the B operand: k-slot (step rr, group lg) <-> row 4 lg + rr.
        f32x4 Tb = zero4();
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float a = Ts[(16 * bi + lj) * kPitchF + 16 * bi + 4 * lg + rr];
          Tb = mfma_f32(a, S[rr], Tb);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) Ts[(16 * bi + 4 * lg + rr) * kPitchF + 16 * bj + lj] = -Tb[rr];
      }
      __syncthreads();
    }

    // T' = T diag(beta) as hi/lo bf16 fragments, and P as bf16 fragments.
    for (int task = tid; task < 2 * kFrags * 64; task += 256) {
      const int kind = task / (kFrags * 64);
      const int rem = task - kind * kFrags * 64;
      const int f = rem >> 6, ll = rem & 63;
      const int i = 16 * frag_row_block(f) + (ll & 15);
      const int c0 = 32 * frag_k_step(f) + 8 * (ll >> 4);
      if (kind == 0) {
        u16x8 vh, vl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cc = c0 + e;
          const float t = (cc < i) ? Ts[i * kPitchF + cc] : (cc == i ? 1.f : 0.f);
          __bf16 bh, bl;
          split_hilo(t * Bs[cc], bh, bl);
          vh[e] = bf16_bits(bh);
          vl[e] = bf16_bits(bl);
        }
        *reinterpret_cast<u16x8 *>(R + kRecTpHi + f * kFragBytes + ll * 16) = vh;
        *reinterpret_cast<u16x8 *>(R + kRecTpLo + f * kFragBytes + ll * 16) = vl;
      } else {
        u16x8 vp;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cc = c0 + e;
          const float pv = (cc <= i) ? Sqk[i * kPitchF + cc] * expf(Gs[i] - Gs[cc]) : 0.f;
          vp[e] = bf16_bits(to_bf16(pv));
        }
        *reinterpret_cast<u16x8 *>(R + kRecP + f * kFragBytes + ll * 16) = vp;
      }
    }
    __syncthreads();
  }
}

void launch_chunk_prep(const void *q, const void *k, const float *g, const float *beta,
                       const int32_t *cu, int N, int Hk, int Hv, int64_t nslots, void *rec,
                       void *kcrec, hipStream_t stream) {
  dim3 grid((unsigned)nslots, (unsigned)Hk);
  hipLaunchKernelGGL(chunk_prep_kernel, grid, dim3(256), 0, stream,
                     static_cast<const unsigned short *>(q), static_cast<const unsigned short *>(k),
                     g, beta, cu, N, Hk, Hv, static_cast<uint8_t *>(rec),
                     static_cast<uint8_t *>(kcrec));
}

}  // namespace gdn
