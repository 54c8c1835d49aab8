// gdn_api.hip -- host side of libgdn: argument checks, workspace carve-up and kernel launches.
// Everything is validated before the first enqueue; nothing here allocates, frees or syncs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_device.h"

namespace gdn {
void launch_chunk_prep(const void *q, const void *k, const float *g, const float *beta,
                       const GateArgs *gates, const int32_t *cu, int64_t T, int N, int Hk, int Hv,
                       int64_t nslots, void *rec, uint32_t *norm_part, hipStream_t stream);
hipError_t launch_state_pass(const void *q, const void *k, const void *v, const int32_t *cu,
                             const float *h0, const int32_t *h0_index, int num_h0, void *o, float *hT,
                             const void *rec, int64_t T, int N, int Hk, int Hv, int max_groups,
                             hipStream_t stream, SplitPass sp, const NormOut *norm, bool o_read_next);
void launch_state_scan(const float *phi, const float *bend, const float *h0, const int32_t *h0_index,
                       int num_h0, float *hs, int segs, int Hv, hipStream_t stream);
void launch_chunk_prep_conv(const void *qkv, const void *conv_w, const void *conv_in,
                            const int32_t *state_index, int num_states, const float *g,
                            const float *beta, const GateArgs *gates, const int32_t *cu, int64_t T,
                            int N, int Hk, int Hv, int64_t nslots, void *rec, void *qo, void *ko,
                            void *vo, uint32_t *norm_part, hipStream_t stream);
void launch_mixer_prep(const void *qkv, const void *conv_w, const int32_t *cu, int64_t T, int N,
                       int Hk, int Hv, const void *conv_in, const int32_t *state_index,
                       int num_states, void *q, void *k, void *v, hipStream_t stream);
void launch_conv_window_out(const void *qkv, const int32_t *cu, int N, int C,
                            const void *conv_in, const int32_t *state_index, int num_states,
                            void *conv_out, hipStream_t stream);
void launch_gated_rmsnorm(const void *o, const void *z, const void *norm_w, float eps, int64_t T,
                          int Hv, void *y, hipStream_t stream);
}  // namespace gdn

namespace {

thread_local int g_last_hip_error = 0;

// Workgroups of the state pass that fit at once on the device the stream runs on (one per CU:
// its LDS use allows no more), rounded down to a multiple of 8; cached per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_max_groups[kMaxDevices];
int device_max_groups(hipStream_t stream) {
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int cached = g_max_groups[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess)
    cus = 0;
  const int groups = cus >= 8 ? cus / 8 * 8 : 8;
  if (dev >= 0) g_max_groups[dev].store(groups, std::memory_order_relaxed);
  return groups;
}

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

// GDN_ERR_ALIAS if two outputs overlap, or an output overlaps an input -- except an output that
// is exactly an input named as its in-place partner (same address; same extent by construction).
struct InPlace {
  const void *out, *in;
};
template <size_t NO, size_t NI, size_t NP>
int check_alias(const Range (&outs)[NO], const Range (&ins)[NI], const InPlace (&ok)[NP]) {
  for (size_t a = 0; a < NO; ++a)
    for (size_t b = a + 1; b < NO; ++b)
      if (overlap(outs[a], outs[b])) return GDN_ERR_ALIAS;
  for (const Range &o : outs)
    for (const Range &i : ins) {
      if (!overlap(o, i)) continue;
      bool allowed = false;
      for (const InPlace &e : ok) allowed |= e.out && o.p == i.p && e.out == o.p && e.in == i.p;
      if (!allowed) return GDN_ERR_ALIAS;
    }
  return GDN_OK;
}

// Checks the shape part of a descriptor; fills derived sizes.
struct Shape {
  int64_t T;
  int N, Hk, Hv;
  int64_t nslots;
  size_t rec_bytes;    // one record per (chunk slot, v-head)
  size_t split_bytes;  // state buffers of the time split (one sequence with few heads), or 0
  size_t ws_bytes;     // workspace of the chunk path: records, then the split's buffers
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
  // A single sequence of at least 32 chunks with at most 8 v-heads may be cut along time into 4 or
  // more segments (plan_split); its three state buffers hold kSplitStates states each.
  s.split_bytes = (s.N == 1 && 4 * s.Hv <= gdn::kSplitStates && s.T > 31 * gdn::kChunk)
                      ? 3 * (size_t)gdn::kSplitStates * gdn::kDim * gdn::kDim * 4 : 0;
  s.ws_bytes = s.rec_bytes + s.split_bytes;
  return GDN_OK;
}

int record_hip(hipError_t e) {
  if (e == hipSuccess) return GDN_OK;
  g_last_hip_error = (int)e;
  return GDN_ERR_HIP;
}

enum Stage { kPrep = 1, kPass = 2, kBoth = 3 };

// Initial states: h0 is [rows, Hv, dk, dv]; sequence n reads row index[n] (zeros when outside
// [0, rows)), or row n when index is NULL (then rows == N).
struct StatePool {
  const float *h0;
  int rows;
  const int32_t *index;
};

// Validates the arguments a chunk-path stage reads and writes (unused pointers are ignored).
int check_chunk_args(const gdn_chunk_desc *d, Shape &s, Stage stage, const void *q, const void *k,
                     const void *v, const float *g, const float *beta, const int32_t *cu,
                     StatePool &pool, const void *o, const float *hT) {
  int st = check_shape(d, s);
  if (st != GDN_OK) return st;
  const bool tok = s.T > 0;
  const bool prep = stage & kPrep, pass = stage & kPass;
  if (!cu) return GDN_ERR_NULL;
  if (tok && (!q || !k)) return GDN_ERR_NULL;
  if (tok && prep && (!g || !beta)) return GDN_ERR_NULL;
  if (tok && pass && (!v || !o)) return GDN_ERR_NULL;
  if (pool.index && pool.rows < 1) return GDN_ERR_SHAPE;
  if (!pool.index) pool.rows = s.N;
  const size_t need = s.ws_bytes;
  if (!d->workspace || d->workspace_bytes < need) return GDN_ERR_WORKSPACE;
  if (!prep) g = beta = nullptr;
  if (!pass) v = nullptr, pool = StatePool{nullptr, s.N, nullptr}, o = nullptr, hT = nullptr;

  const size_t qk_b = (size_t)s.T * s.Hk * gdn::kDim * 2, v_b = (size_t)s.T * s.Hv * gdn::kDim * 2;
  const size_t gb_b = (size_t)s.T * s.Hv * 4, row_b = (size_t)s.Hv * gdn::kDim * gdn::kDim * 4;
  const size_t cu_b = (size_t)(s.N + 1) * 4, idx_b = (size_t)s.N * 4;
  const void *a16[] = {q, k, v, o, pool.h0, hT, d->workspace};
  for (const void *p : a16)
    if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
  const void *a4[] = {g, beta, cu, pool.index};
  for (const void *p : a4)
    if (p && !aligned(p, 4)) return GDN_ERR_ALIGN;

  // The workspace is written by the prep stage and only read by the pass stage.  hT may be h0
  // itself when sequence n reads row n; with an index another sequence may still read the row.
  const Range outs[] = {{o, tok ? v_b : 0}, {hT, s.N * row_b}, {d->workspace, need}};
  const Range ins[] = {{q, qk_b},    {k, qk_b}, {v, v_b},
                       {g, gb_b},    {beta, gb_b}, {cu, cu_b},
                       {pool.h0, (size_t)pool.rows * row_b}, {pool.index, idx_b}};
  const InPlace ok[] = {{pool.index ? nullptr : hT, pool.h0}};
  return check_alias(outs, ins, ok);
}

// The time split: one sequence of nc chunks whose Hv x 8 work items leave most of the device idle
// is cut into segs segments of m chunks (segs x Hv x 8 <= the device's workgroups, segs x Hv <=
// kSplitStates, at least 8 chunks a segment).  The state pass then runs three times over all
// segments at once -- end states from zero states, transitions (v = 0 from the identity), and the
// outputs from each segment's true initial state -- with a scan of the states in between, instead
// of once over nc chunks on a few CUs: about 3 / segs of the chunk steps.  It is planned only with
// at least 4 segments; otherwise segs is 0 and the pass runs as usual.
gdn::SplitPass plan_split(const Shape &s, int max_groups) {
  gdn::SplitPass sp{0, 0, 0, nullptr, nullptr};
  if (!s.split_bytes || s.T <= 0) return sp;
  const int nc = (int)((s.T + gdn::kChunk - 1) / gdn::kChunk);
  int segs = max_groups / (s.Hv * gdn::kDvTiles);
  segs = segs < gdn::kSplitStates / s.Hv ? segs : gdn::kSplitStates / s.Hv;
  segs = segs < nc / 8 ? segs : nc / 8;
  if (segs < 4) return sp;
  sp.m = (nc + segs - 1) / segs;
  sp.segs = (nc + sp.m - 1) / sp.m;
  return sp;
}

// Enqueues the checked stages.  With norm (the mixer's fused gated RMSNorm, planned by the caller
// only where fused_norm_ok holds) the pass writes y instead of o, and the prep marks the row sums
// of squares as not yet written.
int run_chunk(const Shape &s, Stage stage, const void *q, const void *k, const void *v,
              const float *g, const float *beta, const int32_t *cu, const StatePool &pool, void *o,
              float *hT, void *ws, hipStream_t stream, const gdn::NormOut *norm = nullptr,
              const gdn::GateArgs *gates = nullptr, bool o_read_next = false) {
  unsigned char *rec = static_cast<unsigned char *>(ws);
  (void)hipGetLastError();  // clear a stale error so that only our launches are reported
  if ((stage & kPrep) && s.T > 0) {
    gdn::launch_chunk_prep(q, k, g, beta, gates, cu, s.T, s.N, s.Hk, s.Hv, s.nslots, rec,
                           norm ? norm->part : nullptr, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_hip(e);
  }
  if (stage & kPass) {
    const int groups = device_max_groups(stream);
    gdn::SplitPass sp = plan_split(s, groups);
    if (sp.segs) {
      // workspace after the records: end states | transitions | initial states of the segments
      float *bend = reinterpret_cast<float *>(rec + s.rec_bytes);
      float *phi = bend + (size_t)gdn::kSplitStates * gdn::kDim * gdn::kDim;
      float *hs = phi + (size_t)gdn::kSplitStates * gdn::kDim * gdn::kDim;
      if (norm) return GDN_ERR_UNSUPPORTED;  // never planned (fused_norm_ok)
      sp.mode = 0;
      sp.h_out = bend;
      hipError_t e = gdn::launch_state_pass(q, k, v, cu, nullptr, nullptr, 0, o, nullptr, rec, s.T, s.N, s.Hk,
                                            s.Hv, groups, stream, sp, nullptr, false);
      if (e != hipSuccess) return record_hip(e);
      sp.mode = 1;
      sp.h_out = phi;
      e = gdn::launch_state_pass(q, k, v, cu, nullptr, nullptr, 0, o, nullptr, rec, s.T, s.N, s.Hk, s.Hv,
                                 groups, stream, sp, nullptr, false);
      if (e != hipSuccess) return record_hip(e);
      gdn::launch_state_scan(phi, bend, pool.h0, pool.index, pool.rows, hs, sp.segs, s.Hv, stream);
      e = hipGetLastError();
      if (e != hipSuccess) return record_hip(e);
      sp.mode = 2;
      sp.h_in = hs;
      sp.h_out = nullptr;
      return record_hip(gdn::launch_state_pass(q, k, v, cu, nullptr, nullptr, 0, o, hT, rec, s.T, s.N, s.Hk,
                                               s.Hv, groups, stream, sp, nullptr, o_read_next));
    }
    return record_hip(gdn::launch_state_pass(q, k, v, cu, pool.h0, pool.index, pool.rows, o, hT, rec, s.T,
                                             s.N, s.Hk, s.Hv, groups, stream, sp, norm, o_read_next));
  }
  return GDN_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Scratch of gdn_chunk_fwd_noalloc: the chunk path's workspace (records, time-split states) for
// callers that cannot allocate.  Every GPU that loads the library holds its own copy of this
// array until the process ends.  In host code `scratch` names a host-side stand-in, not a device
// address: only the per-device address from hipGetSymbolAddress ever reaches a kernel.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the stream's device's copy of `scratch`, looked up once per device with
// that device current (the caller's current device is restored).  A failed lookup is kept and
// reported on every later call for that device.
int scratch_address(hipStream_t stream, void **out) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return record_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    hipError_t err = hipGetDevice(&cur);
    if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
    void *p = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    g_scratch_ptr[dev] = err == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = err;
  });
  if (g_scratch_err[dev] != hipSuccess) return record_hip(g_scratch_err[dev]);
  *out = g_scratch_ptr[dev];
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
    case GDN_ERR_SCRATCH_LIMIT:
      return "GDN_ERR_SCRATCH_LIMIT: the shape needs more than the static scratch of gdn_chunk_fwd_noalloc";
    default: return "unknown gdn status";
  }
}

int gdn_last_hip_error(void) { return g_last_hip_error; }

size_t gdn_chunk_fwd_workspace_size(const gdn_chunk_desc *d) {
  Shape s;
  if (check_shape(d, s) != GDN_OK) return 0;
  return s.ws_bytes;
}

int gdn_chunk_fwd(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                  const float *g, const float *beta, const int32_t *cu_seqlens, const float *h0,
                  void *o, float *hT, void *stream) {
  Shape s;
  StatePool pool{h0, 0, nullptr};
  const int st = check_chunk_args(d, s, kBoth, q, k, v, g, beta, cu_seqlens, pool, o, hT);
  if (st != GDN_OK) return st;
  return run_chunk(s, kBoth, q, k, v, g, beta, cu_seqlens, pool, o, hT, d->workspace,
                   static_cast<hipStream_t>(stream));
}

int gdn_chunk_fwd_noalloc(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const int32_t *cu_seqlens,
                          const float *h0, void *o, float *hT, void *stream) {
  Shape s;
  int st = check_shape(d, s);
  if (st != GDN_OK) return st;
  if (s.ws_bytes > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH_LIMIT;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  st = scratch_address(strm, &ws);
  if (st != GDN_OK) return st;
  gdn_chunk_desc dd = *d;
  dd.workspace = ws;
  dd.workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
  StatePool pool{h0, 0, nullptr};
  st = check_chunk_args(&dd, s, kBoth, q, k, v, g, beta, cu_seqlens, pool, o, hT);
  if (st != GDN_OK) return st;
  return run_chunk(s, kBoth, q, k, v, g, beta, cu_seqlens, pool, o, hT, ws, strm);
}

int gdn_chunk_fwd_indexed(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                          const float *g, const float *beta, const int32_t *cu_seqlens,
                          const float *h0, int32_t num_h0, const int32_t *h0_index, void *o,
                          float *hT, void *stream) {
  if (!d) return GDN_ERR_NULL;
  if (!h0 || !h0_index) return GDN_ERR_NULL;
  if (num_h0 < 1) return GDN_ERR_SHAPE;
  Shape s;
  StatePool pool{h0, num_h0, h0_index};
  const int st = check_chunk_args(d, s, kBoth, q, k, v, g, beta, cu_seqlens, pool, o, hT);
  if (st != GDN_OK) return st;
  return run_chunk(s, kBoth, q, k, v, g, beta, cu_seqlens, pool, o, hT, d->workspace,
                   static_cast<hipStream_t>(stream));
}

int gdn_chunk_prep(const gdn_chunk_desc *d, const void *q, const void *k, const float *g,
                   const float *beta, const int32_t *cu_seqlens, void *stream) {
  Shape s;
  StatePool pool{nullptr, 0, nullptr};
  const int st = check_chunk_args(d, s, kPrep, q, k, nullptr, g, beta, cu_seqlens, pool,
                                  nullptr, nullptr);
  if (st != GDN_OK) return st;
  return run_chunk(s, kPrep, q, k, nullptr, g, beta, cu_seqlens, pool, nullptr, nullptr,
                   d->workspace, static_cast<hipStream_t>(stream));
}

int gdn_state_pass(const gdn_chunk_desc *d, const void *q, const void *k, const void *v,
                   const int32_t *cu_seqlens, const float *h0, void *o, float *hT,
                   void *stream) {
  Shape s;
  StatePool pool{h0, 0, nullptr};
  const int st = check_chunk_args(d, s, kPass, q, k, v, nullptr, nullptr, cu_seqlens, pool, o, hT);
  if (st != GDN_OK) return st;
  return run_chunk(s, kPass, q, k, v, nullptr, nullptr, cu_seqlens, pool, o, hT, d->workspace,
                   static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
// Mixer: K0 (conv + SiLU + split + q/k L2 norm) -> chunk path -> K4 (gated RMSNorm); with Hv / Hk
// even, K0 is done inside the chunk prep kernel.
// Workspace: [chunk path | q' | k' | v' | o] with the prepped q/k/v and o in bf16.
// ---------------------------------------------------------------------------------------------
namespace {
struct MixerLayout {
  Shape s;
  size_t chunk_bytes, q_bytes, v_bytes, part_bytes, total;
};
int mixer_layout(const gdn_mixer_desc *d, MixerLayout &m) {
  if (!d) return GDN_ERR_NULL;
  int st = check_shape(&d->chunk, m.s);
  if (st != GDN_OK) return st;
  if (d->conv_taps != 4) return GDN_ERR_UNSUPPORTED;
  if (!(d->norm_eps > 0.f)) return GDN_ERR_UNSUPPORTED;
  if (2 * (int64_t)m.s.Hk + m.s.Hv > 65535) return GDN_ERR_SHAPE;  // head segments on grid y
  if ((m.s.T * m.s.Hv + 15) / 16 > INT32_MAX) return GDN_ERR_SHAPE;  // gated RMSNorm grid x
  m.chunk_bytes = m.s.ws_bytes;
  m.q_bytes = round_up((size_t)m.s.T * m.s.Hk * gdn::kDim * 2);
  m.v_bytes = round_up((size_t)m.s.T * m.s.Hv * gdn::kDim * 2);
  m.part_bytes = round_up((size_t)m.s.T * m.s.Hv * gdn::kDvTiles * 4);  // fused norm's row sums
  m.total = m.chunk_bytes + 2 * m.q_bytes + 2 * m.v_bytes + m.part_bytes;
  return GDN_OK;
}

// Whether the mixer's gated RMSNorm can run fused into the state pass: every work item in one round
// of resident workgroups (no persistent walk, no time split) and cooperative launch available.
std::atomic<int> g_coop[kMaxDevices];  // 0 unknown, 1 yes, 2 no
bool fused_norm_ok(const Shape &s, hipStream_t stream) {
  if (s.T <= 0) return false;
  const int groups = device_max_groups(stream);
  if ((int64_t)s.N * s.Hv * gdn::kDvTiles > groups || plan_split(s, groups).segs) return false;
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  int c = g_coop[dev].load(std::memory_order_relaxed);
  if (!c) {
    int coop = 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) coop = 0;
    c = coop ? 1 : 2;
    g_coop[dev].store(c, std::memory_order_relaxed);
  }
  return c == 1;
}
}  // namespace

size_t gdn_mixer_fwd_workspace_size(const gdn_mixer_desc *d) {
  MixerLayout m;
  if (mixer_layout(d, m) != GDN_OK) return 0;
  return m.total;
}

}  // extern "C"

namespace {
// The mixer, with the gated RMSNorm as its own kernel after the state pass (fuse_norm false) or
// fused into the state pass's output path (true; GDN_ERR_UNSUPPORTED where fused_norm_ok fails).
// gates: g and beta made from the projections (gdn_mixer_fwd_gates; g and beta are then unused).
int run_mixer(const gdn_mixer_desc *d, const void *qkv, const void *conv_w, const float *g,
              const float *beta, const gdn::GateArgs *gates, const void *z, const void *norm_w,
              const int32_t *cu_seqlens,
              const float *h0, const void *conv_in, int32_t num_states, const int32_t *state_index,
              void *y, float *hT, void *conv_out, void *stream, bool fuse_norm_requested) {
  MixerLayout m;
  int st = mixer_layout(d, m);
  if (st != GDN_OK) return st;
  const Shape &s = m.s;
  const bool tok = s.T > 0;
  if (!cu_seqlens) return GDN_ERR_NULL;
  if (tok && (!qkv || !conv_w || !z || !norm_w || !y)) return GDN_ERR_NULL;
  if (tok && !gates && (!g || !beta)) return GDN_ERR_NULL;
  if (tok && gates && (!gates->a || !gates->b || !gates->A_log || !gates->dt_bias)) return GDN_ERR_NULL;
  const gdn::GateArgs ga = gates ? *gates : gdn::GateArgs{};
  if (num_states < 1 || (!state_index && num_states != s.N)) return GDN_ERR_SHAPE;
  void *ws = d->chunk.workspace;
  if (!ws || d->chunk.workspace_bytes < m.total) return GDN_ERR_WORKSPACE;

  const int W = d->conv_taps - 1;
  const size_t C = (size_t)(2 * s.Hk + s.Hv) * gdn::kDim;
  const size_t qkv_b = (size_t)s.T * C * 2, cw_b = C * 4 * 2, z_b = (size_t)s.T * s.Hv * gdn::kDim * 2;
  const size_t gb_b = (size_t)s.T * s.Hv * 4, row_b = (size_t)s.Hv * gdn::kDim * gdn::kDim * 4;
  const size_t cu_b = (size_t)(s.N + 1) * 4, nw_b = gdn::kDim * 2, win_b = (size_t)W * C * 2;
  const void *a16[] = {qkv, z, norm_w, y, h0, hT, ws, conv_in, conv_out};
  for (const void *p : a16)
    if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
  const void *a8[] = {conv_w};
  for (const void *p : a8)
    if (p && !aligned(p, 8)) return GDN_ERR_ALIGN;
  const void *a4[] = {g, beta, cu_seqlens, state_index, ga.A_log, ga.dt_bias};
  for (const void *p : a4)
    if (p && !aligned(p, 4)) return GDN_ERR_ALIGN;
  const void *a2[] = {ga.a, ga.b};
  for (const void *p : a2)
    if (p && !aligned(p, 2)) return GDN_ERR_ALIGN;

  // In place (hT == h0, conv_out == conv_in) only when sequence n continues from state n.
  const Range outs[] = {{y, tok ? z_b : 0}, {hT, s.N * row_b}, {conv_out, s.N * win_b},
                        {ws, m.total}};
  const Range ins[] = {{qkv, qkv_b},       {conv_w, cw_b},
                       {g, gb_b},          {beta, gb_b},
                       {z, z_b},           {norm_w, nw_b},
                       {cu_seqlens, cu_b}, {h0, (size_t)num_states * row_b},
                       {conv_in, (size_t)num_states * win_b}, {state_index, (size_t)s.N * 4},
                       {ga.a, (size_t)s.T * s.Hv * 2},     {ga.b, (size_t)s.T * s.Hv * 2},
                       {ga.A_log, (size_t)s.Hv * 4},       {ga.dt_bias, (size_t)s.Hv * 4}};
  const InPlace ok[] = {{state_index ? nullptr : hT, h0}, {state_index ? nullptr : conv_out, conv_in}};
  st = check_alias(outs, ins, ok);
  if (st != GDN_OK) return st;

  hipStream_t strm = static_cast<hipStream_t>(stream);
  unsigned char *base = static_cast<unsigned char *>(ws);
  unsigned char *qp = base + m.chunk_bytes;
  unsigned char *kp = qp + m.q_bytes;
  unsigned char *vp = kp + m.q_bytes;
  unsigned char *op = vp + m.v_bytes;
  uint32_t *part = reinterpret_cast<uint32_t *>(op + m.v_bytes);
  const bool fuse_norm = fuse_norm_requested && tok;
  if (fuse_norm && !fused_norm_ok(s, strm)) return GDN_ERR_UNSUPPORTED;
  const gdn::NormOut norm{static_cast<const unsigned short *>(z), static_cast<const unsigned short *>(norm_w),
                          static_cast<unsigned short *>(y), part, d->norm_eps};
  (void)hipGetLastError();
  // With pairs of v-heads per k-head the chunk prep makes q, k, v from qkv itself (one kernel
  // instead of the input prep, then the chunk prep); otherwise the input prep runs first.
  const bool fused = tok && (s.Hv / s.Hk) % 2 == 0;
  if (fused) {
    gdn::launch_chunk_prep_conv(qkv, conv_w, conv_in, state_index, num_states, g, beta, gates, cu_seqlens,
                                s.T, s.N, s.Hk, s.Hv, s.nslots, base, qp, kp, vp,
                                fuse_norm ? part : nullptr, strm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_hip(e);
  } else if (tok) {
    gdn::launch_mixer_prep(qkv, conv_w, cu_seqlens, s.T, s.N, s.Hk, s.Hv, conv_in, state_index,
                           num_states, qp, kp, vp, strm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_hip(e);
  }
  // after the prep, which reads conv_in: conv_out may be conv_in itself
  if (conv_out) {
    gdn::launch_conv_window_out(qkv, cu_seqlens, s.N, (int)C, conv_in, state_index, num_states,
                                conv_out, strm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return record_hip(e);
  }
  const StatePool pool{h0, num_states, state_index};
  // o is read back by the gated RMSNorm right after the pass: cached stores leave it in L2
  st = run_chunk(s, fused ? kPass : kBoth, qp, kp, vp, g, beta, cu_seqlens, pool, op, hT, base, strm,
                 fuse_norm ? &norm : nullptr, gates, true);
  if (st != GDN_OK) return st;
  if (tok && !fuse_norm) {
    gdn::launch_gated_rmsnorm(op, z, norm_w, d->norm_eps, s.T, s.Hv, y, strm);
    return record_hip(hipGetLastError());
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_mixer_fwd_cont(const gdn_mixer_desc *d, const void *qkv, const void *conv_w,
                       const float *g, const float *beta, const void *z, const void *norm_w,
                       const int32_t *cu_seqlens, const float *h0, const void *conv_in,
                       int32_t num_states, const int32_t *state_index, void *y, float *hT,
                       void *conv_out, void *stream) {
  return run_mixer(d, qkv, conv_w, g, beta, nullptr, z, norm_w, cu_seqlens, h0, conv_in, num_states,
                   state_index, y, hT, conv_out, stream, false);
}

int gdn_mixer_fwd(const gdn_mixer_desc *d, const void *qkv, const void *conv_w, const float *g,
                  const float *beta, const void *z, const void *norm_w,
                  const int32_t *cu_seqlens, const float *h0, void *y, float *hT, void *stream) {
  if (!d) return GDN_ERR_NULL;
  return run_mixer(d, qkv, conv_w, g, beta, nullptr, z, norm_w, cu_seqlens, h0, nullptr, d->chunk.num_seqs,
                   nullptr, y, hT, nullptr, stream, false);
}

int gdn_mixer_fwd_fused_norm(const gdn_mixer_desc *d, const void *qkv, const void *conv_w,
                             const float *g, const float *beta, const void *z, const void *norm_w,
                             const int32_t *cu_seqlens, const float *h0, void *y, float *hT,
                             void *stream) {
  if (!d) return GDN_ERR_NULL;
  return run_mixer(d, qkv, conv_w, g, beta, nullptr, z, norm_w, cu_seqlens, h0, nullptr, d->chunk.num_seqs,
                   nullptr, y, hT, nullptr, stream, true);
}

int gdn_mixer_fwd_gates(const gdn_mixer_desc *d, const void *qkv, const void *conv_w, const void *a,
                        const void *b, const float *A_log, const float *dt_bias, const void *z,
                        const void *norm_w, const int32_t *cu_seqlens, const float *h0, void *y,
                        float *hT, void *stream) {
  if (!d) return GDN_ERR_NULL;
  const gdn::GateArgs ga{static_cast<const unsigned short *>(a), static_cast<const unsigned short *>(b),
                         A_log, dt_bias};
  return run_mixer(d, qkv, conv_w, nullptr, nullptr, &ga, z, norm_w, cu_seqlens, h0, nullptr,
                   d->chunk.num_seqs, nullptr, y, hT, nullptr, stream, false);
}

int gdn_mixer_fwd_gates_cont(const gdn_mixer_desc *d, const void *qkv, const void *conv_w, const void *a,
                             const void *b, const float *A_log, const float *dt_bias, const void *z,
                             const void *norm_w, const int32_t *cu_seqlens, const float *h0,
                             const void *conv_in, int32_t num_states, const int32_t *state_index,
                             void *y, float *hT, void *conv_out, void *stream) {
  const gdn::GateArgs ga{static_cast<const unsigned short *>(a), static_cast<const unsigned short *>(b),
                         A_log, dt_bias};
  return run_mixer(d, qkv, conv_w, nullptr, nullptr, &ga, z, norm_w, cu_seqlens, h0, conv_in, num_states,
                   state_index, y, hT, conv_out, stream, false);
}

}  // extern "C"
