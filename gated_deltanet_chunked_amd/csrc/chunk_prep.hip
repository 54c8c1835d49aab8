// chunk_prep.hip -- state-independent work of every 64-token chunk, all chunks in parallel.
//
// The fused kernel of the "open-jev-fast" README ("Phase 3", item 1) walks a path's chunks one
// by one, and for two-chunk paths computes everything that does not involve the recurrent state
// for both chunks at once.  This kernel takes that split to every chunk: the decay prefix sums,
// the key Gram products, the triangular inverse and the record derived from them, for every
// (chunk, v-head) in parallel; the sequential part lives in state_pass.hip.
//
// One workgroup per (chunk slot, HP = 1 or 2 v-heads of one k-head), 8 waves per v-head.  Every
// v-head of a k-head shares K K^T and Q K^T (only the decays and beta tell them apart), so a pair
// of them shares the products and the q/k loads:
//   1. G = inclusive cumsum of g over the chunk per v-head (a wave64 scan: 64 tokens = 64 lanes).
//   2. S = K K^T and Q K^T over the lower 16x16 block triangle on bf16 MFMA (fp32 accumulate),
//      each block computed transposed, so that a lane holds 4 consecutive columns of one row.
//   3. From the accumulators, per v-head:
//        A_ij = beta_i e^{G_i - G_j} (k_i . k_j)  for i > j      (fp32, LDS)
//        P_ij = e^{G_i - G_j} (q_i . k_j)         for i >= j     (bf16, straight to the record)
//      Off the diagonal blocks the decay is a product of two tabulated factors,
//      e^{G_i - G_r} e^{G_r - G_j} with r the first token of i's 16-row block (j < r <= i, so both
//      exponents are <= 0); only the diagonal blocks take one exponential per entry.
//   4. T = (I + A)^-1: each 16x16 diagonal block by right-looking substitution (four lanes per
//      column), then block column j by T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj on fp32 MFMA, with
//      the column's blocks kept in registers, one wave per block column (no barrier in between).
//   5. T' = T diag(beta) as bf16 hi + lo MFMA fragments, e^{G} and e^{G_last - G}: the rest of the
//      record the state pass reads.
// The record's T' fragments and decays are written with streaming (non-temporal) stores: only the
// next kernel reads them, often from another XCD, so they should be in memory when this kernel ends
// rather than written back from L2 at the kernel boundary; P, whose lanes are written in two
// halves, goes through L2.
// Every exponent is <= 0 (G is non-increasing), so no e^{-G} is ever formed.  Tokens past the
// end of a sequence enter as k = q = 0, g = 0, beta = 0, which leaves T' and P zero on them.
#include "gdn_device.h"

namespace gdn {

namespace {

constexpr int kPitchF = 68;                        // fp32 row pitch of 64 x 64 LDS matrices
// Records of at most this many bytes in all are written with cached stores, so that the state pass,
// which reads them next, finds them in L2; larger ones, which cannot all stay there, with
// streaming stores (measured both ways at T = 16,384: cached stores made the prep 1.2 us faster
// and the pass 1.1 us slower).  P is always cached: its 16-byte pieces are written in two halves
// by different waves and merge in L2.
constexpr uint64_t kRecStreamBytes = 16u << 20;
template <typename V>
__device__ __forceinline__ void rec_store(V *p, V v, bool nt) {
  if (nt) __builtin_nontemporal_store(v, p);
  else *p = v;
}
constexpr int kMatBytes = kChunk * kPitchF * 4;    // 17408
constexpr int kMaxHeads = 2;                       // v-heads per workgroup
// LDS map: [Ks | Qs] (bf16 64 x 128, swizzled) are dead once the products are in registers, so
// the A matrices reuse their space; then the T matrices, then G and beta per v-head.
constexpr int kOffKs = 0;
constexpr int kOffQs = kChunk * kDim * 2;                  // 16384
constexpr int kOffA = 0;                                   // + x * kMatBytes
constexpr int kOffT = kMaxHeads * kMatBytes;               // 34816 + x * kMatBytes
constexpr int kOffG = 2 * kMaxHeads * kMatBytes;           // 69632: G[x][64]
constexpr int kOffB = kOffG + kMaxHeads * kChunk * 4;      // beta[x][64]
// Decay factors: Er[x][i] = e^{G_i - G_{16 (i / 16)}}; Fc[x][rb - 1][j] = e^{G_{16 rb} - G_j} for
// j < 16 rb, rb = 1..3.
constexpr int kOffEr = kOffB + kMaxHeads * kChunk * 4;
constexpr int kOffFc = kOffEr + kMaxHeads * kChunk * 4;
// Conv weights of the four 128-channel blocks (q, k, v, v; 4 taps, bf16) when the kernel makes q,
// k, v itself.
constexpr int kOffW = kOffFc + kMaxHeads * 3 * kChunk * 4;
constexpr int kLdsBytes = kOffW + 4 * kDim * 4 * 2;  // 76800 with the conv weights, 72704 without: two workgroups per CU
static_assert(kMaxHeads * kMatBytes >= 2 * kChunk * kDim * 2, "the A matrices cover Ks and Qs");

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The value of lane 4 (l / 4) + q (lane q of this lane's quad), through a DPP quad permutation;
// q must fold to a constant (the DPP control is an immediate).
__device__ __forceinline__ float quad_bcast(float v, int q) {
  const int b = __float_as_int(v);
  switch (q) {
    case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x00, 0xF, 0xF, false));
    case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x55, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xAA, 0xF, 0xF, false));
    default: return __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0xFF, 0xF, 0xF, false));
  }
}

// Byte offset of bf16 element (row, col) in a swizzled 64 x 128 tile: 16-byte chunks are
// XOR-permuted by row so that 16 lanes reading one chunk column of 16 rows hit distinct banks.
__device__ __forceinline__ int swz(int row, int col) {
  return row * (kDim * 2) + ((((col >> 3) ^ (row & 15))) << 4) + ((col & 7) << 1);
}

// Floor of the per-token log-decay.  Every decay used is e^{G_i - G_j}, a difference of fp32
// cumsums inside the chunk, accurate to about one ulp of |G|; one token with a huge |g| (say -1e5,
// a decay far below any fp32 resolution) would leave the later differences of the chunk with errors
// of order one in the exponent.  A decay of e^-40 (4e-18) per token already wipes the state out to
// below fp32 resolution of anything it is added to, so g is floored there: |G| <= 64 x 40 and the
// differences stay within ~2e-4 of the exact ones, while no result changes visibly.
constexpr float kLogDecayFloor = -40.f;

// e^x for x <= 0 from the hardware 2^x (v_exp_f32): relative error about 1e-7 |x|.
__device__ __forceinline__ float exp_neg(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// hi = bf16(x), lo = bf16(x - hi) for two values at once (packed bf16 pairs).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// Largest n in [0, N) with cu[n] / 64 + n <= slot (that map is increasing in n).  One round of
// 64 lanes per 64 sequences; every wave runs it, results are wave-uniform.
__device__ __forceinline__ int find_sequence(const int32_t *__restrict__ cu, int N, int slot, int l) {
  int n = 0;
  for (int b0 = 0; b0 < N; b0 += 64) {
    const int idx = b0 + l;
    const bool ok = idx < N && (cu[idx] / kChunk + idx) <= slot;
    const unsigned long long m = __ballot(ok);
    if (m == 0ull) break;
    n = b0 + 63 - __clzll(m);
    if (~m != 0ull) break;
  }
  return n;
}

// Record fragment holding row block rb, token step ks (see gdn_device.h).
__device__ __forceinline__ int frag_index(int rb, int ks) { return rb < 2 ? rb : 2 * rb - 2 + ks; }

// Lower-triangle block b (0..9) -> (row block, column block), column block <= row block.
__device__ __forceinline__ int block_row(int b) { return b < 1 ? 0 : (b < 3 ? 1 : (b < 6 ? 2 : 3)); }

}  // namespace

// The GDN mixer's input prep done by the prep kernel itself (kConv): q, k, v from the packed
// q | k | v input by a causal depthwise conv (4 taps, the carried window before a sequence start)
// and SiLU, q and k L2-normalized per head -- the arithmetic of mixer_prep_kernel, token by token.
// The workgroup of (slot, v-heads 2 p, 2 p + 1) makes the chunk's q and k of their k-head and v of
// both v-heads, writes them for the state pass and keeps q, k in LDS for its own products.
struct ConvArgs {
  const unsigned short *qkv, *conv_w, *conv_in;
  const int32_t *state_index;
  int num_states;
  unsigned short *qo, *ko, *vo;
};

// HP v-heads per workgroup, kWavesPerHead waves per v-head: the products, the A/P scaling and the
// T' fragments spread over all of them; the diagonal solve and the column chains run on the first
// 4 waves of each head.
constexpr int kWavesPerHead = 8;
// kGates: g and beta made from the projections (ga), else read as given.
template <int HP, bool kConv, bool kGates>
__global__ __launch_bounds__(64 * kWavesPerHead * HP) void chunk_prep_kernel(
    const unsigned short *__restrict__ q, const unsigned short *__restrict__ k,
    const float *__restrict__ g, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, int T, int N, int Hk, int Hv, uint8_t *__restrict__ rec,
    ConvArgs ca, GateArgs ga, uint32_t *__restrict__ norm_part, bool rec_nt) {
  static_assert(!kConv || HP == 2, "the input prep runs on pairs of v-heads");
  constexpr int kThreads = 64 * kWavesPerHead * HP, kWaves = kWavesPerHead * HP;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kConv ? kLdsBytes : kOffW];
  unsigned char *Ks = smem + kOffKs;
  unsigned char *Qs = smem + kOffQs;
  float *Gall = reinterpret_cast<float *>(smem + kOffG);
  float *Ball = reinterpret_cast<float *>(smem + kOffB);
  float *Erall = reinterpret_cast<float *>(smem + kOffEr);
  float *Fcall = reinterpret_cast<float *>(smem + kOffFc);

  // Workgroup b runs on XCD b % 8.  For one sequence the state pass keeps v-heads
  // [x Hv / 8, (x + 1) Hv / 8) on XCD x; dealing the (slot, head group) units out the same way puts
  // each head's prep on the XCD (and L2) that reads its q and k next.  An XCD takes its head
  // groups slot by slot, so the groups of one slot run together and share, in L2, the g and beta
  // lines (one line holds every v-head of a token) and, with more than two v-heads per k-head, q
  // and k.
  int slot = blockIdx.x, grp = blockIdx.y;
  if (N == 1 && gridDim.y % 8 == 0) {
    const int bid = blockIdx.y * gridDim.x + blockIdx.x, per = gridDim.y / 8, j = bid / 8;
    slot = j / per;
    grp = (bid % 8) * per + j % per;
  }
  const int h_first = grp * HP, hk = h_first / (Hv / Hk);
  const int tid = threadIdx.x, l = tid & 63, lj = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w / kWavesPerHead, wl = w % kWavesPerHead;  // v-head within the group, wave within it
  const int h = h_first + hh;

  int tb = 0, te = T, n = 0;
  if (N > 1) {
    n = find_sequence(cu, N, slot, l);
    tb = cu[n];
    te = cu[n + 1];
  }
  const int c = slot - (tb / kChunk + n);
  const int t0 = tb + kChunk * c;
  if (t0 >= te) return;  // slot unused (uniform across the workgroup)
  const int L = min(kChunk, te - t0);
  uint8_t *const rec_slot = rec + (size_t)slot * Hv * kRecBytes;  // v-head x at + x * kRecBytes
  // With the gated RMSNorm fused into the state pass: mark this chunk's row sums of squares of
  // the group's v-heads as not yet written (one word per thread: 64 rows x HP heads x 8 tiles).
  if (norm_part) {
    const int r = tid / (HP * kDvTiles), x = (tid / kDvTiles) % HP, tile = tid % kDvTiles;
    if (r < L) norm_part[((size_t)(t0 + r) * Hv + h_first + x) * kDvTiles + tile] = kPartEmpty;
  }
  static_assert(kThreads == kChunk * HP * kDvTiles, "one word of norm_part per thread");

  // ---- 1. global loads up front; gate cumsum per v-head --------------------------------------
  // The first wave loads the gates (or their inputs) of the workgroup's v-heads -- adjacent in each
  // row, one load per token for both -- together with its q/k loads (every wave loading its own
  // head's gates, once the q/k data had arrived, took 79.2 us at T = 16,384 against 66.8), and
  // later makes their cumsums, decay tables and record decays.
  const size_t gi = (size_t)(t0 + min(l, L - 1)) * Hv + h_first;
  float g_raw[HP] = {}, b_raw[HP] = {};
  GateIn gin[HP] = {};
  auto load_gates = [&]() {
    if (w != 0) return;
    if constexpr (kGates) {
#pragma unroll
      for (int x = 0; x < HP; ++x) gin[x] = gate_load(ga, gi + x, h_first + x);
    } else if constexpr (HP == 2) {
      const f32x2 g2 = *reinterpret_cast<const f32x2 *>(g + gi), b2 = *reinterpret_cast<const f32x2 *>(beta + gi);
      g_raw[0] = g2[0], g_raw[1] = g2[1], b_raw[0] = b2[0], b_raw[1] = b2[1];
    } else {
      g_raw[0] = g[gi];
      b_raw[0] = beta[gi];
    }
  };
  constexpr int kIt = 1024 / kThreads;  // 16-byte pieces of one 64 x 128 tile per thread
  if constexpr (kConv) {
    // Waves 4 b .. 4 b + 3 make block b of the four 128-channel blocks q, k (k-head hk), v (v-heads
    // h_first, h_first + 1); thread (token group tg, 8-channel group cg) makes channels cg * 8 .. + 7
    // of tokens t0 + 4 tg .. + 3 from the 7 input rows its taps slide over.  Lanes 16 m .. 16 m + 15
    // share a token group, so the L2 norm is a 16-lane butterfly.  With more than two v-heads per
    // k-head the k-head's first pair writes q and k.  All input rows are loaded before anything is
    // stored (the stores could alias the input for all the compiler knows), and the blocks' conv
    // weights go through LDS once.
    constexpr int kTok = 4;
    const int blk = w >> 2, tl = tid & 255, tg = tl >> 4, cg = tl & 15;
    const int C = (2 * Hk + Hv) * kDim;
    auto seg_of = [&](int b) { return b == 0 ? hk : (b == 1 ? Hk + hk : 2 * Hk + h_first + b - 2); };
    unsigned short *Ws = reinterpret_cast<unsigned short *>(smem + kOffW);
    const int tfirst = t0 + kTok * tg;
    const unsigned short *win =
        tfirst - 3 < tb ? window_of(ca.conv_in, ca.state_index, ca.num_states, n, (size_t)3 * C) : nullptr;
    const int ch0 = seg_of(blk) * kDim + cg * 8;
    const int tend = t0 + L;  // rows at or past it serve no token of this chunk
    u16x8 xr[kTok + 3];
    bool hv[kTok + 3];
#pragma unroll
    for (int i = 0; i < kTok + 3; ++i) {
      const int src = tfirst - 3 + i;
      hv[i] = src < tend && (src >= tb || win);
      const unsigned short *row = src >= tb ? ca.qkv + (size_t)src * C : win + (size_t)(src - tb + 3) * C;
      if (hv[i]) xr[i] = *reinterpret_cast<const u16x8 *>(row + ch0);
    }
    // The weights after the rows: loaded and stored to LDS first, behind a branch that the
    // compiler does not move the row loads above, they made the rows wait one memory round trip.
    if (tid < 4 * kDim) {  // 8 bytes per thread: the 4 taps of one channel
      const int b = tid / kDim, ch = tid % kDim;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2 *>(Ws + (b * kDim + ch) * 4) =
          *reinterpret_cast<const u32x2 *>(ca.conv_w + (size_t)(seg_of(b) * kDim + ch) * 4);
    }
    __syncthreads();  // the conv weights are in LDS
    float wt[8][4];
    {
      const u16x8 *wp = reinterpret_cast<const u16x8 *>(Ws + (blk * kDim + cg * 8) * 4);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const u16x8 wv = wp[e2];  // taps of channels 2 e2, 2 e2 + 1
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wt[2 * e2][j] = bits_to_float(wv[j]);
          wt[2 * e2 + 1][j] = bits_to_float(wv[4 + j]);
        }
      }
    }
    const bool write_qk = (h_first / 2) % ((Hv / Hk) / 2) == 0;
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int r = kTok * tg + u, t = t0 + r;
      const bool valid = r < L;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      if (valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (hv[u + j]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += wt[e][j] * bits_to_float(xr[u + j][e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = silu(acc[e]);
      }
      if (blk < 2) {
        float ss2 = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss2 += acc[e] * acc[e];
        ss2 = sum16(ss2);
        const float rn = rsqrt_hw(ss2 + 1e-6f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= rn;
      }
      u16x8 out;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = bf16_bits(to_bf16(acc[e]));
      if (valid && (blk >= 2 || write_qk)) {
        unsigned short *dst = blk == 0   ? ca.qo + ((size_t)t * Hk + hk) * kDim
                              : blk == 1 ? ca.ko + ((size_t)t * Hk + hk) * kDim
                                         : ca.vo + ((size_t)t * Hv + h_first + blk - 2) * kDim;
        *reinterpret_cast<u16x8 *>(dst + cg * 8) = out;
      }
      if (blk < 2)  // zeros past L
        *reinterpret_cast<u16x8 *>((blk == 0 ? Qs : Ks) + r * (kDim * 2) + ((cg ^ (r & 15)) << 4)) = out;
    }
  } else {
    u32x4 kv[kIt], qv[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int p = tid + kThreads * it, row = p >> 4, ch = p & 15;
      const size_t off = ((size_t)(t0 + min(row, L - 1)) * Hk + hk) * kDim + ch * 8;
      kv[it] = *reinterpret_cast<const u32x4 *>(k + off);
      qv[it] = *reinterpret_cast<const u32x4 *>(q + off);
    }
    load_gates();
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int p = tid + kThreads * it, row = p >> 4, ch = p & 15;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const int so = row * (kDim * 2) + ((ch ^ (row & 15)) << 4);
      *reinterpret_cast<u32x4 *>(Ks + so) = row < L ? kv[it] : zero;
      *reinterpret_cast<u32x4 *>(Qs + so) = row < L ? qv[it] : zero;
    }
  }
  if constexpr (kConv) {
    // after the input prep (issued with its row loads, the gate loads measured slower)
    __builtin_amdgcn_sched_barrier(0);
    load_gates();
  }
  if (w == 0) {
    if constexpr (kGates) {
#pragma unroll
      for (int x = 0; x < HP; ++x) gate_values(gin[x], g_raw[x], b_raw[x]);  // from the projections
    }
#pragma unroll
    for (int x = 0; x < HP; ++x) {
      const float gv = l < L ? fmaxf(g_raw[x], kLogDecayFloor) : 0.f;
      const float bv = l < L ? b_raw[x] : 0.f;
      const float G = wave_inclusive_scan(gv);
      const float Glast = lane_value(G, 63);
      const float G16 = lane_value(G, 16), G32 = lane_value(G, 32), G48 = lane_value(G, 48);
      // Er: G relative to the first token of this lane's 16-row block
      const float Gr = (l >> 4) == 0 ? lane_value(G, 0) : (l >> 4) == 1 ? G16 : (l >> 4) == 2 ? G32 : G48;
      Gall[kChunk * x + l] = G;
      Ball[kChunk * x + l] = bv;
      Erall[kChunk * x + l] = exp_neg(G - Gr);
      // Fc[rb - 1][j] = e^{G_{16 rb} - G_j} for j < 16 rb
      Fcall[kChunk * (3 * x + 0) + l] = l < 16 ? exp_neg(G16 - G) : 0.f;
      Fcall[kChunk * (3 * x + 1) + l] = l < 32 ? exp_neg(G32 - G) : 0.f;
      Fcall[kChunk * (3 * x + 2) + l] = l < 48 ? exp_neg(G48 - G) : 0.f;
      uint8_t *R = rec_slot + (size_t)(h_first + x) * kRecBytes;
      rec_store(reinterpret_cast<float *>(R + kRecEG) + l, exp_neg(G), rec_nt);
      rec_store(reinterpret_cast<float *>(R + kRecED) + l, exp_neg(Glast - G), rec_nt);
    }
  }
  __syncthreads();

  // ---- 2. block products, transposed: C[j][i] = sum_d K[j][d] X[i][d], X = K (p < 10) or Q ----
  // Block b of the lower triangle is (row block rb, column block cb); accumulator lane (lj, lg)
  // then holds S[i = 16 rb + lj][j = 16 cb + 4 lg + rr], rr = 0..3.
  constexpr int kPer = (20 + kWaves - 1) / kWaves;
  f32x4 acc[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int p = w + kWaves * it;
    if (p < 20) {
      const int which = p >= 10 ? 1 : 0;
      const int b = p - 10 * which;
      const int rb = block_row(b), cb = b - rb * (rb + 1) / 2;
      const unsigned char *Xm = which ? Qs : Ks;
      acc[it] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = 4 * ks + lg;
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Ks + swz(16 * cb + lj, ch * 8));
        const bf16x8 bx = *reinterpret_cast<const bf16x8 *>(Xm + swz(16 * rb + lj, ch * 8));
        acc[it] = mfma_bf16(a, bx, acc[it]);
      }
    }
  }
  __syncthreads();  // Ks, Qs are dead from here on; the A matrices take their space

  // ---- 3. A (fp32, LDS) and P (bf16 record fragments) for every v-head of the group -----------
  // P's fragment k-slots follow the accumulators: fragment (rb, ks), lane (i, g) slot e holds
  // P[i][32 ks + 16 (e / 4) + 4 g + e % 4], so block (rb, cb) fills bytes 8 (cb % 2) .. + 7 of each
  // lane's 16 bytes, and the zero block beside a diagonal block is written as zeros.
  // A's off-diagonal blocks are stored row-major; its diagonal blocks (read only by the
  // substitution, which walks columns) are stored transposed: entry (o + a, o + b) holds A[o+b][o+a].
  // A diagonal block of K K^T is symmetric, so the same accumulator gives both.
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const int p = w + kWaves * it;
    if (p < 20) {
      const int which = p >= 10 ? 1 : 0;
      const int b = p - 10 * which;
      const int rb = block_row(b), cb = b - rb * (rb + 1) / 2;
      const int i = 16 * rb + lj, j0 = 16 * cb + 4 * lg;
#pragma unroll
      for (int x = 0; x < HP; ++x) {
        const float *Gx = Gall + kChunk * x;
        // Decays e^{G_i - G_j}, j = j0 .. j0 + 3: tabulated factors off the diagonal blocks.
        f32x4 e;
        if (rb != cb) {
          const float ei = Erall[kChunk * x + i];
          const f32x4 fj = *reinterpret_cast<const f32x4 *>(Fcall + kChunk * (3 * x + rb - 1) + j0);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) e[rr] = ei * fj[rr];
        }
        if (which) {
          float d[4];
          if (rb != cb) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) d[rr] = e[rr] * acc[it][rr];
          } else {
            const float Gi = Gx[i];
            const f32x4 Gj = *reinterpret_cast<const f32x4 *>(Gx + j0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) d[rr] = j0 + rr <= i ? exp_neg(Gi - Gj[rr]) * acc[it][rr] : 0.f;
          }
          const u32x2 val = {pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3])};
          uint8_t *dst = rec_slot + (size_t)(h_first + x) * kRecBytes + kRecP +
                         frag_index(rb, cb >> 1) * kFragBytes + l * 16 + 8 * (cb & 1);
          // Cached stores: the two 8-byte halves of a lane's 16 bytes come from different waves and
          // merge in L2 before the line goes to memory (streaming stores would send each half-line
          // on its own: 23 MB more written at T = 16,384).
          if ((cb & 1) == 0 && cb + 1 > rb) {  // the other half is an upper block: zeros
            const u32x4 v4 = {val[0], val[1], 0u, 0u};
            *reinterpret_cast<u32x4 *>(dst) = v4;
          } else {
            *reinterpret_cast<u32x2 *>(dst) = val;
          }
        } else {
          float *Ax = reinterpret_cast<float *>(smem + kOffA + x * kMatBytes);
          f32x4 av;
          if (rb != cb) {
            const float bi = Ball[kChunk * x + i];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) av[rr] = bi * e[rr] * acc[it][rr];
          } else {
            const float Gi = Gx[i];
            const f32x4 Gj = *reinterpret_cast<const f32x4 *>(Gx + j0);
            const f32x4 bj = *reinterpret_cast<const f32x4 *>(Ball + kChunk * x + j0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              av[rr] = j0 + rr > i ? bj[rr] * exp_neg(Gj[rr] - Gi) * acc[it][rr] : 0.f;
          }
          *reinterpret_cast<f32x4 *>(Ax + i * kPitchF + j0) = av;
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. T = (I + A)^-1 for this wave's v-head ------------------------------------------------
  const float *As = reinterpret_cast<const float *>(smem + kOffA + hh * kMatBytes);
  float *Ts = reinterpret_cast<float *>(smem + kOffT + hh * kMatBytes);
  // Diagonal block wl by right-looking substitution on all 64 lanes: lane 4 cj + r holds rows
  // 4 r .. 4 r + 3 of column cj of the block's inverse.  Step m broadcasts x_m (row m, held by
  // lane 4 cj + m / 4) across the lane quad and subtracts A[i][m] x_m from every row i; A[i][m]
  // is 0 for i <= m (A is strictly lower), so no row needs masking.  The 15 columns of A that the
  // steps use sit contiguously in the transposed diagonal-block storage and are read up front.
  if (wl < 4) {
    const int o = 16 * wl, cj = l >> 2, r = l & 3;
    f32x4 ac[15];  // ac[m][e] = A[o + 4 r + e][o + m]
#pragma unroll
    for (int m = 0; m < 15; ++m) ac[m] = *reinterpret_cast<const f32x4 *>(As + (o + m) * kPitchF + o + 4 * r);
    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = 4 * r + e == cj ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; ++m) {
      const float xm = quad_bcast(x[m % 4], m / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] -= ac[m][e] * xm;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Ts[(o + 4 * r + e) * kPitchF + o + cj] = x[e];
  }
  __syncthreads();

  // Block column j = wl: T_ij = -T_ii S_i, S_i = sum_{m=j}^{i-1} A_im T_mj for i = j + 1 .. 3.
  // Every S_i starts with its T_jj term (independent of the chain); each new T_ij is then folded
  // into the S of the rows below it at once, so the dependent chain is one product by T_ii and one
  // by A per block.  All operands are read from LDS before the chain starts and the results are
  // stored after it, so no LDS access waits inside the chain.  The column's blocks stay in
  // registers (C layout: lane (col lj, rows 4 lg + rr)); in every product the k-slot (step s,
  // lane group lg) stands for row 4 lg + s of the B operand, so an accumulator is fed back as B
  // without moving data between lanes.
  // Wave w runs on SIMD w % 4; the second v-head takes the block columns in reverse order, so the
  // long chain of column 0 never shares a SIMD's matrix unit with the other head's.
  if (wl < 4) {
    const int j = hh ? 3 - wl : wl;
    // A operands (row lj, cols 4 lg + s): Aj[i] = A_ij, Am[i][m] = A_im (j < m < i), Tii[i] = T_ii;
    // every register array index is a compile-time constant (j is not).
    f32x4 Aj[4], Am[4][4], Tii[4], Tjj;
#pragma unroll
    for (int s = 0; s < 4; ++s) Tjj[s] = Ts[(16 * j + 4 * lg + s) * kPitchF + 16 * j + lj];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (i > j) {
        Tii[i] = *reinterpret_cast<const f32x4 *>(Ts + (16 * i + lj) * kPitchF + 16 * i + 4 * lg);
        Aj[i] = *reinterpret_cast<const f32x4 *>(As + (16 * i + lj) * kPitchF + 16 * j + 4 * lg);
#pragma unroll
        for (int m = 1; m < 3; ++m)
          if (m > j && m < i)
            Am[i][m] = *reinterpret_cast<const f32x4 *>(As + (16 * i + lj) * kPitchF + 16 * m + 4 * lg);
      }
    }
    f32x4 S[4], Tc[4];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      S[i] = zero4();
      if (i > j) {
#pragma unroll
        for (int s = 0; s < 4; ++s) S[i] = mfma_f32(Aj[i][s], Tjj[s], S[i]);
      }
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (i > j) {
        f32x4 Tb = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) Tb = mfma_f32(Tii[i][s], S[i][s], Tb);
#pragma unroll
        for (int s = 0; s < 4; ++s) Tc[i][s] = -Tb[s];
#pragma unroll
        for (int i2 = i + 1; i2 < 4; ++i2) {
#pragma unroll
          for (int s = 0; s < 4; ++s) S[i2] = mfma_f32(Am[i2][i][s], Tc[i][s], S[i2]);
        }
      }
    }
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i > j) {
#pragma unroll
        for (int s = 0; s < 4; ++s) Ts[(16 * i + 4 * lg + s) * kPitchF + 16 * j + lj] = Tc[i][s];
      }
  }
  __syncthreads();

  // ---- 5. T' = T diag(beta) as bf16 hi/lo fragments -------------------------------------------
  // Fragment f, lane ll: row i = 16 rb(f) + ll % 16, columns 32 ks(f) + 8 (ll / 16) .. + 7.  The
  // (v-head, fragment) tasks of the group are dealt over all its waves.
  for (int u = tid; u < HP * kFrags * 64; u += kThreads) {
    const int x = u / (kFrags * 64), task = u - x * (kFrags * 64);
    const int f = task >> 6, ll = task & 63;
    uint8_t *R = rec_slot + (size_t)(h_first + x) * kRecBytes;
    const float *Bh = Ball + kChunk * x;
    const float *Tx = reinterpret_cast<const float *>(smem + kOffT + x * kMatBytes);
    const int i = 16 * frag_row_block(f) + (ll & 15);
    const int c0 = 32 * frag_k_step(f) + 8 * (ll >> 4);
    const f32x4 m0 = *reinterpret_cast<const f32x4 *>(Tx + i * kPitchF + c0);
    const f32x4 m1 = *reinterpret_cast<const f32x4 *>(Tx + i * kPitchF + c0 + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(Bh + c0);
    const f32x4 b1 = *reinterpret_cast<const f32x4 *>(Bh + c0 + 4);
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int cc = c0 + e;
      const float mv = e < 4 ? m0[e] : m1[e - 4];
      const float bb = e < 4 ? b0[e] : b1[e - 4];
      t[e] = cc < i ? mv * bb : (cc == i ? bb : 0.f);
    }
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_pair(t[2 * e], t[2 * e + 1], hv[e], lv[e]);
    const u32x4 vh = {hv[0], hv[1], hv[2], hv[3]}, vl = {lv[0], lv[1], lv[2], lv[3]};
    rec_store(reinterpret_cast<u32x4 *>(R + kRecTpHi + f * kFragBytes + ll * 16), vh, rec_nt);
    rec_store(reinterpret_cast<u32x4 *>(R + kRecTpLo + f * kFragBytes + ll * 16), vl, rec_nt);
  }
}

void launch_chunk_prep(const void *q, const void *k, const float *g, const float *beta,
                       const GateArgs *gates, const int32_t *cu, int64_t T, int N, int Hk, int Hv,
                       int64_t nslots, void *rec, uint32_t *norm_part, hipStream_t stream) {
  const GateArgs ga = gates ? *gates : GateArgs{};
  const unsigned short *qp = static_cast<const unsigned short *>(q);
  const unsigned short *kp = static_cast<const unsigned short *>(k);
  uint8_t *rp = static_cast<uint8_t *>(rec);
  const dim3 pairs((unsigned)nslots, (unsigned)(Hv / 2)), singles((unsigned)nslots, (unsigned)Hv);
  const bool rec_nt = (uint64_t)nslots * (uint64_t)Hv * kRecBytes > kRecStreamBytes;
  if ((Hv / Hk) % 2 == 0) {  // pairs of v-heads of one k-head per workgroup
    if (gates)
      hipLaunchKernelGGL((chunk_prep_kernel<2, false, true>), pairs, dim3(128 * kWavesPerHead), 0, stream, qp,
                         kp, g, beta, cu, (int)T, N, Hk, Hv, rp, ConvArgs{}, ga, norm_part, rec_nt);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<2, false, false>), pairs, dim3(128 * kWavesPerHead), 0, stream, qp,
                         kp, g, beta, cu, (int)T, N, Hk, Hv, rp, ConvArgs{}, ga, norm_part, rec_nt);
  } else {
    if (gates)
      hipLaunchKernelGGL((chunk_prep_kernel<1, false, true>), singles, dim3(64 * kWavesPerHead), 0, stream, qp,
                         kp, g, beta, cu, (int)T, N, Hk, Hv, rp, ConvArgs{}, ga, norm_part, rec_nt);
    else
      hipLaunchKernelGGL((chunk_prep_kernel<1, false, false>), singles, dim3(64 * kWavesPerHead), 0, stream, qp,
                         kp, g, beta, cu, (int)T, N, Hk, Hv, rp, ConvArgs{}, ga, norm_part, rec_nt);
  }
}

// The same with q, k, v made from the packed mixer input (Hv / Hk even): writes q, k, v (q/k
// [T, Hk, 128], v [T, Hv, 128], bf16) as the mixer's input prep does, and the records.
void launch_chunk_prep_conv(const void *qkv, const void *conv_w, const void *conv_in,
                            const int32_t *state_index, int num_states, const float *g,
                            const float *beta, const GateArgs *gates, const int32_t *cu, int64_t T,
                            int N, int Hk, int Hv, int64_t nslots, void *rec, void *qo, void *ko,
                            void *vo, uint32_t *norm_part, hipStream_t stream) {
  const ConvArgs ca{static_cast<const unsigned short *>(qkv), static_cast<const unsigned short *>(conv_w),
                    static_cast<const unsigned short *>(conv_in), state_index, num_states,
                    static_cast<unsigned short *>(qo), static_cast<unsigned short *>(ko),
                    static_cast<unsigned short *>(vo)};
  const dim3 grid((unsigned)nslots, (unsigned)(Hv / 2));
  const bool rec_nt = (uint64_t)nslots * (uint64_t)Hv * kRecBytes > kRecStreamBytes;
  const unsigned short *none = nullptr;
  if (gates)
    hipLaunchKernelGGL((chunk_prep_kernel<2, true, true>), grid, dim3(128 * kWavesPerHead), 0, stream, none,
                       none, g, beta, cu, (int)T, N, Hk, Hv, static_cast<uint8_t *>(rec), ca, *gates, norm_part, rec_nt);
  else
    hipLaunchKernelGGL((chunk_prep_kernel<2, true, false>), grid, dim3(128 * kWavesPerHead), 0, stream, none,
                       none, g, beta, cu, (int)T, N, Hk, Hv, static_cast<uint8_t *>(rec), ca, GateArgs{}, norm_part, rec_nt);
}

}  // namespace gdn
