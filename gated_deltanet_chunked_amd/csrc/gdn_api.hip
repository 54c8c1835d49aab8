// gdn_api.hip -- host side of libgdn: argument checks, workspace carve-up and kernel launches.
// Everything is validated before the first enqueue; nothing here allocates, frees or syncs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/gdn.h"
#include "gdn_device.h"

namespace gdn {
void launch_chunk_prep(const void *q, const void *k, const float *g, const float *beta,
                       const int32_t *cu, int64_t T, int N, int Hk, int Hv, int64_t nslots,
                       void *rec, hipStream_t stream);
void launch_state_pass(const void *q, const void *k, const void *v, const int32_t *cu,
                       const float *h0, void *o, float *hT, const void *rec, int N, int Hk, int Hv,
                       hipStream_t stream);
void launch_mixer_prep(const void *qkv, const void *conv_w, const int32_t *cu, int64_t T, int N,
                       int Hk, int Hv, void *q, void *k, void *v, hipStream_t stream);
void launch_gated_rmsnorm(const void *o, const void *z, const void *norm_w, float eps, int64_t T,
                          int Hv, void *y, hipStream_t stream);
}  // namespace gdn

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Range {
  const void *p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks the shape part of a descriptor; fills derived sizes.
struct Shape {
  int64_t T;
  int N, Hk, Hv;
  int64_t nslots;
  size_t rec_bytes;  // workspace of the chunk path: one record per (chunk slot, v-head)
};

int check_shape(const gdn_chunk_desc *d, Shape &s) {
  if (!d) return GDN_ERR_NULL;
  if (d->head_dim_k != gdn::kDim || d->head_dim_v != gdn::kDim) return GDN_ERR_UNSUPPORTED;
  if (d->num_seqs < 1 || d->total_tokens < 0 || d->num_k_heads < 1 || d->num_v_heads < 1)
    return GDN_ERR_SHAPE;
  if (d->num_v_heads % d->num_k_heads != 0) return GDN_ERR_SHAPE;
  if (d->total_tokens > INT32_MAX - 2 * gdn::kChunk || d->num_v_heads > 65535) return GDN_ERR_SHAPE;
  const int64_t blocks = (int64_t)d->num_seqs * d->num_v_heads * gdn::kDvTiles;
  if (blocks > INT32_MAX) return GDN_ERR_SHAPE;
  s.T = d->total_tokens;
  s.N = d->num_seqs;
  s.Hk = d->num_k_heads;
  s.Hv = d->num_v_heads;
  s.nslots = gdn::num_slots(s.T, s.N);
  if (s.nslots > INT32_MAX) return GDN_ERR_SHAPE;
  s.rec_bytes = round_up((size_t)s.nslots * s.Hv * gdn::kRecBytes);
  return GDN_OK;
}

int record_hip(hipError_t e) {
  if (e == hipSuccess) return GDN_OK;
  g_last_hip_error = (int)e;
  return GDN_ERR_HIP;
}

enum Stage { kPrep = 1, kPass = 2, kBoth = 3 };

// Validates the arguments a chunk-path stage reads and writes (unused pointers are ignored).
int check_chunk_args(const gdn_chunk_desc *d, Shape &s, Stage stage, const void *q, const void *k,
                     const void *v, const float *g, const float *beta, const int32_t *cu,
                     const float *h0, const void *o, const float *hT) {
  int st = check_shape(d, s);
  if (st != GDN_OK) return st;
  const bool tok = s.T > 0;
  const bool prep = stage & kPrep, pass = stage & kPass;
  if (!cu) return GDN_ERR_NULL;
  if (tok && (!q || !k)) return GDN_ERR_NULL;
  if (tok && prep && (!g || !beta)) return GDN_ERR_NULL;
  if (tok && pass && (!v || !o)) return GDN_ERR_NULL;
  const size_t need = s.rec_bytes;
  if (!d->workspace || d->workspace_bytes < need) return GDN_ERR_WORKSPACE;
  if (!prep) g = beta = nullptr;
  if (!pass) v = nullptr, h0 = nullptr, o = nullptr, hT = nullptr;

  const size_t qk_b = (size_t)s.T * s.Hk * gdn::kDim * 2, v_b = (size_t)s.T * s.Hv * gdn::kDim * 2;
  const size_t gb_b = (size_t)s.T * s.Hv * 4, st_b = (size_t)s.N * s.Hv * gdn::kDim * gdn::kDim * 4;
  const size_t cu_b = (size_t)(s.N + 1) * 4;
  const void *a16[] = {q, k, v, o, h0, hT, d->workspace};
  for (const void *p : a16)
    if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
  const void *a4[] = {g, beta, cu};
  for (const void *p : a4)
    if (p && !aligned(p, 4)) return GDN_ERR_ALIGN;

  // The workspace is written by the prep stage and only read by the pass stage.
  const Range ins[] = {{q, qk_b}, {k, qk_b}, {v, v_b}, {g, gb_b}, {beta, gb_b}, {cu, cu_b}};
  const Range ro{o, tok ? v_b : 0}, rh{hT, st_b}, rw{d->workspace, need}, rh0{h0, st_b};
  for (const Range &in : ins)
    if (overlap(ro, in) || overlap(rh, in) || overlap(rw, in)) return GDN_ERR_ALIAS;
  if (overlap(ro, rh) || overlap(ro, rw) || overlap(rh, rw) || overlap(ro, rh0) || overlap(rw, rh0))
    return GDN_ERR_ALIAS;
  if (hT && h0 && hT != h0 && overlap(rh, rh0)) return GDN_ERR_ALIAS;
  return GDN_OK;
}

// Enqueues the checked stages.
int run_chunk(const Shape &s, Stage stage, const void *q, const void *k, const void *v,
              const float *g, const float *beta, const int32_t *cu, const float *h0, void *o,
              float *hT, void *ws, hipStream_t stream) {
  unsigned char *rec = static_cast<unsigned char *>(ws);
  (void)hipGetLastError();  // clear a stale error so that only our launches are reported
  if ((stage & kPrep) && s.T > 0) {
    gdn::launch_chunk_prep(q, k, g, beta, cu, s.T, s.N, s.Hk, s.Hv, s.nslots, rec, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_hip(e);
  }
  if (stage & kPass) {
    gdn::launch_state_pass(q, k, v, cu, h0, o, hT, rec, s.N, s.Hk, s.Hv, stream);
    return record_hip(hipGetLastError());
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK: enqueued";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: invalid sizes (N, T, Hk, Hv) or size overflow";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dims other than 128 or unsupported option";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer not aligned as required";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps an input or the workspace";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: a HIP launch failed (see gdn_last_hip_error)";
    default: return "unknown gdn status";
  }
}

int gdn_last_hip_error(void) { return g_last_hip_error; }

size_t gdn_chunk_fwd_workspace_size(const gdn_chunk_desc *d) {
  Shape s;
  if (check_shape(d, s) != GDN_OK) return 0;
  return s.rec_bytes;
}

int gdn_chunk_fwd(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                  const float *g, const float *beta, const int32_t *cu_seqlens, const float *h0,
                  void *o, float *hT, void *stream) {
  Shape s;
  const int st = check_chunk_args(d, s, kBoth, q, k, v, g, beta, cu_seqlens, h0, o, hT);
  if (st != GDN_OK) return st;
  return run_chunk(s, kBoth, q, k, v, g, beta, cu_seqlens, h0, o, hT, d->workspace,
                   static_cast<hipStream_t>(stream));
}

int gdn_chunk_prep(const gdn_chunk_desc *d, const void *q, const void *k, const float *g,
                   const float *beta, const int32_t *cu_seqlens, void *stream) {
  Shape s;
  const int st = check_chunk_args(d, s, kPrep, q, k, nullptr, g, beta, cu_seqlens, nullptr,
                                  nullptr, nullptr);
  if (st != GDN_OK) return st;
  return run_chunk(s, kPrep, q, k, nullptr, g, beta, cu_seqlens, nullptr, nullptr, nullptr,
                   d->workspace, static_cast<hipStream_t>(stream));
}

int gdn_state_pass(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                   const int32_t *cu_seqlens, const float *h0, void *o, float *hT,
                   void *stream) {
  Shape s;
  const int st = check_chunk_args(d, s, kPass, q, k, v, nullptr, nullptr, cu_seqlens, h0, o, hT);
  if (st != GDN_OK) return st;
  return run_chunk(s, kPass, q, k, v, nullptr, nullptr, cu_seqlens, h0, o, hT, d->workspace,
                   static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
// Mixer: K0 (conv + SiLU + split + q/k L2 norm) -> chunk path -> K4 (gated RMSNorm).
// Workspace: [chunk path | q' | k' | v' | o] with the prepped q/k/v and o in bf16.
// ---------------------------------------------------------------------------------------------
namespace {
struct MixerLayout {
  Shape s;
  size_t chunk_bytes, q_bytes, v_bytes, total;
};
int mixer_layout(const gdn_mixer_desc *d, MixerLayout &m) {
  if (!d) return GDN_ERR_NULL;
  int st = check_shape(&d->chunk, m.s);
  if (st != GDN_OK) return st;
  if (d->conv_taps != 4) return GDN_ERR_UNSUPPORTED;
  if (!(d->norm_eps > 0.f)) return GDN_ERR_UNSUPPORTED;
  if ((int64_t)(2 * m.s.Hk + m.s.Hv) * gdn::kDim > INT32_MAX / 2) return GDN_ERR_SHAPE;
  m.chunk_bytes = m.s.rec_bytes;
  m.q_bytes = round_up((size_t)m.s.T * m.s.Hk * gdn::kDim * 2);
  m.v_bytes = round_up((size_t)m.s.T * m.s.Hv * gdn::kDim * 2);
  m.total = m.chunk_bytes + 2 * m.q_bytes + 2 * m.v_bytes;
  return GDN_OK;
}
}  // namespace

size_t gdn_mixer_fwd_workspace_size(const gdn_mixer_desc *d) {
  MixerLayout m;
  if (mixer_layout(d, m) != GDN_OK) return 0;
  return m.total;
}

int gdn_mixer_fwd(const gdn_mixer_desc *d, const void *qkv, const void *conv_w, const float *g,
                  const float *beta, const void *z, const void *norm_w,
                  const int32_t *cu_seqlens, const float *h0, void *y, float *hT, void *stream) {
  MixerLayout m;
  int st = mixer_layout(d, m);
  if (st != GDN_OK) return st;
  const Shape &s = m.s;
  const bool tok = s.T > 0;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (tok && (!qkv || !conv_w || !g || !beta || !z || !norm_w || !y)) return GDN_ERR_NULL;
  void *ws = d->chunk.workspace;
  if (!ws || d->chunk.workspace_bytes < m.total) return GDN_ERR_WORKSPACE;

  const size_t C = (size_t)(2 * s.Hk + s.Hv) * gdn::kDim;
  const size_t qkv_b = (size_t)s.T * C * 2, cw_b = C * 4 * 2, z_b = (size_t)s.T * s.Hv * gdn::kDim * 2;
  const size_t gb_b = (size_t)s.T * s.Hv * 4, st_b = (size_t)s.N * s.Hv * gdn::kDim * gdn::kDim * 4;
  const size_t cu_b = (size_t)(s.N + 1) * 4, nw_b = gdn::kDim * 2;
  const void *a16[] = {qkv, z, norm_w, y, h0, hT, ws};
  for (const void *p : a16)
    if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
  const void *a8[] = {conv_w};
  for (const void *p : a8)
    if (p && !aligned(p, 8)) return GDN_ERR_ALIGN;
  const void *a4[] = {g, beta, cu_seqlens};
  for (const void *p : a4)
    if (p && !aligned(p, 4)) return GDN_ERR_ALIGN;

  const Range ins[] = {{qkv, qkv_b}, {conv_w, cw_b}, {g, gb_b}, {beta, gb_b},
                       {z, z_b},     {norm_w, nw_b}, {cu_seqlens, cu_b}};
  const Range ry{y, tok ? z_b : 0}, rh{hT, st_b}, rw{ws, m.total}, rh0{h0, st_b};
  for (const Range &in : ins) {
    if (overlap(ry, in) || overlap(rh, in) || overlap(rw, in)) return GDN_ERR_ALIAS;
  }
  if (overlap(ry, rh) || overlap(ry, rw) || overlap(rh, rw) || overlap(ry, rh0) || overlap(rw, rh0))
    return GDN_ERR_ALIAS;
  if (hT && h0 && hT != h0 && overlap(rh, rh0)) return GDN_ERR_ALIAS;

  hipStream_t strm = static_cast<hipStream_t>(stream);
  unsigned char *base = static_cast<unsigned char *>(ws);
  unsigned char *qp = base + m.chunk_bytes;
  unsigned char *kp = qp + m.q_bytes;
  unsigned char *vp = kp + m.q_bytes;
  unsigned char *op = vp + m.v_bytes;
  (void)hipGetLastError();
  if (tok) {
    gdn::launch_mixer_prep(qkv, conv_w, cu_seqlens, s.T, s.N, s.Hk, s.Hv, qp, kp, vp, strm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_hip(e);
  }
  st = run_chunk(s, kBoth, qp, kp, vp, g, beta, cu_seqlens, h0, op, hT, base, strm);
  if (st != GDN_OK) return st;
  if (tok) {
    gdn::launch_gated_rmsnorm(op, z, norm_w, d->norm_eps, s.T, s.Hv, y, strm);
    return record_hip(hipGetLastError());
  }
  return GDN_OK;
}

}  // extern "C"
