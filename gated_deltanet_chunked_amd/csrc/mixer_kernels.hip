// mixer_kernels.hip -- the GDN layer's input prep and output norm around the chunked rule.
//
// The "open-jev-fast" README ("Phase 2", item 1) has one fused kernel for the work before the
// Gated DeltaNet rule (the convolution, its SiLU, the q/k/v split and normalisation) and one for
// the gated norm after it; by "Phase 3" item 3 q and k stay at the 16 key heads.  Both kernels
// here are HBM-bound streams: 16-byte vector loads and stores, fp32 math (SiLU and the norms'
// reciprocal square roots on the hardware exp2 / rcp / rsq units: the outputs are bf16), and the
// per-row reductions as 16-lane butterflies inside a wave (no LDS).
#include "gdn_device.h"

namespace gdn {

// Grid: (ceil(T / (16 kPrepTokens)), 2 Hk + Hv).  Block y selects a 128-channel head segment of
// the packed q | k | v channels; each thread owns 8 channels x kPrepTokens consecutive tokens.
// Lanes 16m .. 16m+15 of a wave hold the 16 channel groups of the same tokens, so the per-token
// L2 norm is a 16-lane butterfly.
//
// A thread loads the kPrepTokens + 3 input rows its conv window slides over all at once (one
// round trip to memory instead of one per tap), and finds the sequence of each of its tokens by
// binary searches over cu_seqlens run side by side.  Positions before a sequence's first token
// read the carried window (conv_in, [3, C] per state), or zeros when there is none.
constexpr int kPrepTokens = 2;

__global__ __launch_bounds__(256) void mixer_prep_kernel(
    const unsigned short *__restrict__ qkv, const unsigned short *__restrict__ conv_w,
    const int32_t *__restrict__ cu, int T, int N, int Hk, int Hv,
    const unsigned short *__restrict__ conv_in, const int32_t *__restrict__ state_index,
    int num_states, unsigned short *__restrict__ qo, unsigned short *__restrict__ ko,
    unsigned short *__restrict__ vo) {
  constexpr int P = kPrepTokens;
  const int seg = blockIdx.y;                  // 0..Hk-1: q heads, Hk..2Hk-1: k heads, then v heads
  const int C = (2 * Hk + Hv) * kDim;
  const int tid = threadIdx.x, chg = tid & 15, tg = tid >> 4;  // channel group, token group
  const int ch0 = seg * kDim + chg * 8;
  const bool is_qk = seg < 2 * Hk;
  const int t0 = (blockIdx.x * 16 + tg) * P;

  // input rows t0 - 3 .. t0 + P - 1, clamped into [0, T - 1]: a clamped row is never used
  // (a row before 0 or before a sequence start fails src >= ss; a row past T - 1 only serves
  // tokens past the end)
  u16x8 xr[P + 3];
#pragma unroll
  for (int r = 0; r < P + 3; ++r) {
    const int row = min(max(t0 - 3 + r, 0), T - 1);
    xr[r] = *reinterpret_cast<const u16x8 *>(qkv + (size_t)row * C + ch0);
  }

  // conv weights of my 8 channels: w[ch][0..3], tap 3 multiplies the current token
  float wt[8][4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
    const u16x4 wv = *reinterpret_cast<const u16x4 *>(conv_w + (size_t)(ch0 + e) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[e][j] = bits_to_float(wv[j]);
  }

  // sequence of token t0 + u: the largest n with cu[n] <= t (cu[0] = 0); ss = cu[n].  Every
  // search runs the same ceil(log2 N) steps; each step halves the range [lo, hi].
  int lo[P], hi[P], ss[P];
#pragma unroll
  for (int u = 0; u < P; ++u) lo[u] = 0, hi[u] = N - 1, ss[u] = 0;
  const int steps = N > 1 ? 32 - __clz(N - 1) : 0;
  for (int st = 0; st < steps; ++st) {
    int mid[P], cm[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
      mid[u] = (lo[u] + hi[u] + 1) >> 1;  // lo <= mid <= hi <= N - 1
      cm[u] = cu[mid[u]];
    }
#pragma unroll
    for (int u = 0; u < P; ++u) {
      if (lo[u] < hi[u]) {
        if (cm[u] <= t0 + u) lo[u] = mid[u], ss[u] = cm[u];
        else hi[u] = mid[u] - 1;
      }
    }
  }

#pragma unroll
  for (int u = 0; u < P; ++u) {
    const int t = t0 + u;
    const bool valid = t < T;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (valid) {
      const unsigned short *win =
          t - 3 < ss[u] ? window_of(conv_in, state_index, num_states, lo[u], (size_t)3 * C) : nullptr;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = t - 3 + j;
        u16x8 xv;
        bool have = true;
        if (src >= ss[u]) xv = xr[u + j];
        else if (win) xv = *reinterpret_cast<const u16x8 *>(win + (size_t)(src - ss[u] + 3) * C + ch0);
        else have = false;
        if (have) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += wt[e][j] * bits_to_float(xv[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = silu(acc[e]);
    }
    if (is_qk) {
      float ss2 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss2 += acc[e] * acc[e];
      ss2 = sum16(ss2);
      const float rn = rsqrt_hw(ss2 + 1e-6f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= rn;
    }
    if (valid) {
      u16x8 out;
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = bf16_bits(to_bf16(acc[e]));
      unsigned short *dst;
      if (seg < Hk) dst = qo + ((size_t)t * Hk + seg) * kDim;
      else if (seg < 2 * Hk) dst = ko + ((size_t)t * Hk + (seg - Hk)) * kDim;
      else dst = vo + ((size_t)t * Hv + (seg - 2 * Hk)) * kDim;
      *reinterpret_cast<u16x8 *>(dst + chg * 8) = out;
    }
  }
}

// y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z), one (token, v-head) row of 128 per 16 lanes.
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(
    const unsigned short *__restrict__ o, const unsigned short *__restrict__ z,
    const unsigned short *__restrict__ norm_w, float eps, int64_t rows,
    unsigned short *__restrict__ y) {
  const int tid = threadIdx.x, chg = tid & 15;
  const int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4);
  const bool valid = row < rows;
  const size_t off = (size_t)(valid ? row : 0) * kDim + chg * 8;
  const u16x8 ov = *reinterpret_cast<const u16x8 *>(o + off);
  const u16x8 zv = *reinterpret_cast<const u16x8 *>(z + off);
  const u16x8 wv = *reinterpret_cast<const u16x8 *>(norm_w + chg * 8);
  // z and the weights are used only under the store's branch, and the compiler would sink their
  // loads into it, behind the wait for o and the row sum: one more memory round trip.  Used here,
  // all three loads are in flight together.
  asm volatile("" ::"v"(zv), "v"(wv));
  float of[8], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    of[e] = bits_to_float(ov[e]);
    ss += of[e] * of[e];
  }
  ss = sum16(ss);
  const float r = rsqrt_hw(ss * (1.f / kDim) + eps);
  u16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float zf = bits_to_float(zv[e]);
    out[e] = bf16_bits(to_bf16(of[e] * r * bits_to_float(wv[e]) * silu(zf)));
  }
  if (valid) *reinterpret_cast<u16x8 *>(y + off) = out;
}

// conv_out[n] = the last 3 rows of sequence n's input stream (its carried window, or zeros,
// followed by its tokens), bit for bit.  Grid (N, ceil(C / 8 / 256)); a thread moves 8 channels
// of all 3 rows and reads them all before it writes, so conv_out may be conv_in itself when
// sequence n reads window n.
__global__ __launch_bounds__(256) void conv_window_out_kernel(
    const unsigned short *__restrict__ qkv, const int32_t *__restrict__ cu, int C,
    const unsigned short *conv_in, const int32_t *__restrict__ state_index, int num_states,
    unsigned short *conv_out) {
  const int n = blockIdx.x;
  const int ch = 8 * (blockIdx.y * 256 + threadIdx.x);
  if (ch >= C) return;
  const int tb = cu[n], te = cu[n + 1];
  const unsigned short *win = window_of(conv_in, state_index, num_states, n, (size_t)3 * C);
  u16x8 rows[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int p = te - 3 + j;  // stream position, >= tb - 3
    const unsigned short *x = p >= tb ? qkv + (size_t)p * C
                              : win   ? win + (size_t)(p - tb + 3) * C
                                      : nullptr;
    if (x) {
      rows[j] = *reinterpret_cast<const u16x8 *>(x + ch);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) rows[j][e] = 0;
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
    *reinterpret_cast<u16x8 *>(conv_out + ((size_t)n * 3 + j) * C + ch) = rows[j];
}

void launch_mixer_prep(const void *qkv, const void *conv_w, const int32_t *cu, int64_t T, int N,
                       int Hk, int Hv, const void *conv_in, const int32_t *state_index,
                       int num_states, void *q, void *k, void *v, hipStream_t stream) {
  dim3 grid((unsigned)((T + 16 * kPrepTokens - 1) / (16 * kPrepTokens)), (unsigned)(2 * Hk + Hv));
  hipLaunchKernelGGL(mixer_prep_kernel, grid, dim3(256), 0, stream,
                     static_cast<const unsigned short *>(qkv),
                     static_cast<const unsigned short *>(conv_w), cu, (int)T, N, Hk, Hv,
                     static_cast<const unsigned short *>(conv_in), state_index, num_states,
                     static_cast<unsigned short *>(q), static_cast<unsigned short *>(k),
                     static_cast<unsigned short *>(v));
}

void launch_conv_window_out(const void *qkv, const int32_t *cu, int N, int C, const void *conv_in,
                            const int32_t *state_index, int num_states, void *conv_out,
                            hipStream_t stream) {
  dim3 grid((unsigned)N, (unsigned)((C / 8 + 255) / 256));
  hipLaunchKernelGGL(conv_window_out_kernel, grid, dim3(256), 0, stream,
                     static_cast<const unsigned short *>(qkv), cu, C,
                     static_cast<const unsigned short *>(conv_in), state_index, num_states,
                     static_cast<unsigned short *>(conv_out));
}

void launch_gated_rmsnorm(const void *o, const void *z, const void *norm_w, float eps, int64_t T,
                          int Hv, void *y, hipStream_t stream) {
  const int64_t rows = T * Hv;
  hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream,
                     static_cast<const unsigned short *>(o), static_cast<const unsigned short *>(z),
                     static_cast<const unsigned short *>(norm_w), eps, rows,
                     static_cast<unsigned short *>(y));
}

}  // namespace gdn
