// state_pass.hip -- the sequential inter-chunk state pass fused with the chunk output.
//
// As in the fused kernel of the "open-jev-fast" README ("Phase 3", item 1), the fp32 recurrent
// state stays on chip and is all that one chunk hands to the next.  Here one workgroup owns one
// (sequence, v-head, 16-column slice of the 128 value columns): the state slice H[:, cols]
// (128 x 16 fp32) lives in MFMA accumulators, spread over 4 compute waves (32 key rows each, see
// state_key), and the chunks of the sequence are walked in order.  Sequences, heads and slices run in parallel.
//
// With H = S^T (key-major), local cumsum G, T' = (I + A)^-1 diag(beta) and
// P = tril(Q K^T o e^{G_i - G_j}) from chunk_prep.hip, one chunk is
//     X  = K H                                   (bf16 K x H split hi/lo: 2 MFMA terms)
//     R  = V - e^{G} o X
//     U~ = T' R                                  (T' and R split hi/lo: 3 MFMA terms)
//     o  = e^{G} o (Q H) + P U~                  (output path in plain bf16)
//     H  = e^{G_last} H + K^T (e^{G_last - G} o U~)   (decayed U~ split hi/lo: 2 MFMA terms)
// which is the chunked form of the gated delta rule: (I + A) U~ = diag(beta)(V - e^G o K H).
// The hi/lo splits keep the state path at about 16 significant bits per operand, so the fp32
// state does not drift over hundreds of chunks even when nothing decays (g = 0, where a bf16 H in
// X alone puts the final state 1.2e-3 off after 256 chunks); bf16 is used where only the output
// sees it (H in Q H, P, U~ in P U~).
//
// A chunk takes three phases, separated by workgroup barriers b1, b2, b3:
//   phase 1: compute waves: X = K H, R = V - e^G o X to LDS (hi/lo)
//            output waves:  o = e^G o (Q H) + P U~ of the previous chunk, staged in LDS -> b1
//   phase 2: compute waves: U~ = T' R (K^T fragments read behind it); U~ (decayed
//            hi/lo and plain) to LDS
//            output waves:  the previous chunk's rows to memory; Q H                 -> b2
//   phase 3: compute waves: H update, H (bf16 hi and lo) to LDS; the next chunk's K rows
//            output waves:  the LDS operands of this chunk's P U~                    -> b3
// Phase 1 ends on the output waves and carries the most LDS traffic, phase 3 the least: the
// reads of phase 3 that are not needed until phase 1 take LDS load off phase 1 (measured: 2-3 %
// off the pass at T = 16,384; reading everything of a phase at once, before its first product,
// was slower).
// so the output path of chunk c finishes during chunk c + 1, off the chunk's last barrier (the
// persistent kernel runs it between b2 and b3 of chunk c instead; see there).
// Thirteen waves per workgroup:
//   * 4 compute waves (one per SIMD) keep the state and do no global access in the chunk loop.
//   * 4 producer waves issue the bulk loads as global->LDS loads (global_load_lds_dwordx4: 1 KiB
//     per instruction, no VGPRs) into a 3-deep ring: the K, Q and V tiles and the record's T'
//     fragments of chunk c + 2 go into the slot chunk c - 1 left, spread over the three phases
//     of chunk c (K before b1, Q before b2, V, the last third of T' and the decays before b3), so
//     no phase waits on a burst of load issue.  Each wave's share is fixed, so the vmcnt
//     bookkeeping is static.
//   * 4 output waves (one per row block) compute the output; each loads its own P fragments
//     straight into registers a chunk ahead and issues no global->LDS loads, so its LDS reads
//     never queue behind its own loads.
//   * 1 prefetch wave pulls every line into L2 six chunks ahead of use, with loads it never waits
//     for, since a miss to HBM takes longer than a chunk.
// LDS carries the tiles and the three cross-wave exchanges per chunk: H, R and U~.
#include "gdn_device.h"

namespace gdn {

namespace {

constexpr int kHtBytes = kDvTile * kDim * 2;    // H exchange buffer (bf16 hi, and again lo)
constexpr int kXBytes = kDvTile * kChunk * 2;    // R / U~ exchange buffers
constexpr int kComputeWaves = 4;
constexpr int kProducerWaves = 4;     // one per SIMD, beside one compute wave
constexpr int kOutputWaves = 4;       // one per SIMD, beside one compute wave
constexpr int kOutputWave0 = kComputeWaves + kProducerWaves;
constexpr int kPrefetchWave = kOutputWave0 + kOutputWaves;
constexpr int kThreads = 64 * (kPrefetchWave + 1);
constexpr int kPrefetchAhead = 6;     // chunks between the L2 warm-up of a chunk and its use
constexpr uint64_t kOStreamBytes = 16u << 20;  // o up to this size: streaming stores (store_o)
// Tile ring slot: K tile | Q tile (64 x 128 bf16 each, swizzled) | V tile (64 x 16 bf16) |
// T' hi and lo fragments of the record (12 KiB, as stored).
constexpr int kTileStages = 3;
constexpr int kTK = 0;
constexpr int kTQ = kTK + kChunk * kDim * 2;              // 16384
constexpr int kTV = kTQ + kChunk * kDim * 2;              // 32768
constexpr int kTT = kTV + kChunk * kDvTile * 2;           // 34816
constexpr int kTpBytes = kRecP - kRecTpHi;                // 12288
constexpr int kTileBytes = kTT + kTpBytes;                // 47104
constexpr int kOBytes = 16 * kDvTile * 2;                 // one row block's 16 output rows
constexpr int kDecBytes = kRecBytes - kRecEG;             // e^G and e^{G_last - G}: 512
constexpr int kDecStages = 3;                             // decay ring slots
constexpr int kDmaTile = kChunk * kDim * 2 / 1024;        // 16 instructions of 1 KiB (K or Q)
constexpr int kDmaV = kChunk * kDvTile * 2 / 1024;        // 2
static_assert(kTileBytes % 16 == 0 && kTV % 16 == 0, "16-byte LDS slots");

// Byte offset of bf16 element (row, col) in a swizzled 64 x 128 tile: 16-byte chunks are
// XOR-permuted by row so that 16 lanes reading one chunk column of 16 rows hit distinct banks.
__device__ __forceinline__ int swz(int row, int col) {
  return row * (kDim * 2) + ((((col >> 3) ^ (row & 15))) << 4) + ((col & 7) << 1);
}

// Value-major exchange buffers (16 value columns x n keys or tokens, bf16) are stored chunk-major:
// the 16-byte chunk holding entries 8c .. 8c + 7 of column j sits at byte 16 (16 c + j).  A lane
// group reading one chunk of columns 0..15 (an MFMA B operand) then touches 256 contiguous bytes,
// which the LDS serves without bank conflicts (padded column-major rows conflict 4-way).
__device__ __forceinline__ int vmaj(int j, int e) { return 16 * (16 * (e >> 3) + j) + 2 * (e & 7); }

// U~ for the P U~ product, in the token order of P's k-slots (chunk_prep.hip writes P straight from
// its accumulators): k-step ks, lane group g holds tokens 32 ks + 4 g .. + 3, then 32 ks + 16 + 4 g
// .. + 3, stored as one 16-byte chunk at byte 16 (16 (4 ks + g) + j) for column j.
__device__ __forceinline__ int pmaj(int j, int t) {
  return 16 * (16 * (4 * (t >> 5) + ((t >> 2) & 3)) + j) + 8 * ((t >> 4) & 1) + 2 * (t & 3);
}

// State rows held by compute wave w: accumulator a, C-layout row i (0..15) is key
// 8 (w + 8 a) + i for i < 8 and 8 (w + 8 a + 4) + i - 8 for i >= 8.  Taking the two 8-key
// chunks of a K^T fragment 4 chunks apart keeps its transposing reads free of bank conflicts
// under the row swizzle of the K tile; every wave still owns 32 keys and the 4 waves all 128.
__device__ __forceinline__ int state_key(int w, int a, int i) {
  return 8 * (w + 8 * a + 4 * (i >> 3)) + (i & 7);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane (buffer_load_dwordx4
// ... lds): a wave-uniform base in a buffer resource (SGPRs) and a 32-bit per-lane byte offset, so
// that moving to the next chunk costs scalar work only.  The compiler's builtins set M0 (the LDS
// base) themselves.  Completion is tracked by this wave's vmcnt only.  Offsets stay below 2^32
// (at most 63 rows of a 16.7 MB row stride); the resource's range (2^32 - 1 bytes) never clips.
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, unsigned lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(sbase), 0, 0xffffffffu, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(uintptr_t)lds, 16, voff, 0, 0, 0);
}
// 4 bytes per lane into a scratch LDS word: pulls the 128-byte line holding src into L2.
__device__ __forceinline__ void touch(const void *src, unsigned lds) {
  __builtin_amdgcn_global_load_lds((global_void *)(uintptr_t)src, (lds_void *)(uintptr_t)lds, 4, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for the waves that issue global->LDS loads (producers, prefetch wave).  The
// compiler sees those loads as outstanding LDS writes, and the workgroup release fence of
// __syncthreads() would make it wait for all of them at every barrier, draining the tile ring.
// These waves publish nothing at a barrier except what their explicit vmcnt waits have already
// made land, so they take the barrier alone, fenced only against compiler reordering.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
__device__ __forceinline__ void store_u32x2(void *dst, uint32_t a, uint32_t b) {
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

// Producers.  Per chunk the four producer waves issue the K and Q tiles (16 instructions each),
// the V tile (2), the T' fragments of the record (12) and its decays (one, half a wave).  Wave
// pw's share is fixed -- tile rows 4m .. 4m + 3 for m = pw mod 4, and the V tile on wave 3 -- so
// the vmcnt bookkeeping is static.  Rows past the sequence end are
// clamped to its last row, which the compute waves never use.
constexpr int kDmaTp = kTpBytes / 1024;                   // 12: T' KiB m on wave m % 4
__host__ __device__ constexpr int kTileCount(int pw) { return 8 + kDmaTp / 4 + (pw == 3 ? kDmaV : 0); }
static_assert(kTileCount(0) + kTileCount(1) + kTileCount(2) + kTileCount(3) ==
                  2 * kDmaTile + kDmaV + kDmaTp, "every load has an owner");
static_assert(kRecTpLo == kRecTpHi + kTpBytes / 2 && kDmaTp % 4 == 0, "T' hi | lo contiguous");
// Producer wave kDecWave also loads the chunk's decays (one half-wave instruction).
constexpr int kDecWave = 1;
__host__ __device__ constexpr int kChunkCount(int pw) { return kTileCount(pw) + (pw == kDecWave ? 1 : 0); }
// Loads every producer wave issues in parts 0 and 1 of a chunk (one T' KiB and four tile rows each).
constexpr int kPartsBeforeB2 = 2 * (1 + 4);

// Per-lane byte offsets of a producer wave's loads, fixed for the whole sequence.  Tile
// instruction i of wave pw covers tile rows 16 i + 4 pw .. + 3 (lane l: row 16 i + 4 pw + l / 16,
// logical 16-byte chunk (l % 16) ^ (row % 16), stored at physical chunk l % 16); the row part
// 16 i and the chunk's first token go into the scalar base.  V instruction m (wave 3) covers
// rows 32 m + l / 2, 8 columns each.
struct ProducerLanes {
  uint32_t tile;  // (4 pw + l / 16) * row stride + 16 * lc
  uint32_t v;     // (l / 2) * Hv * 256 + 2 * (d0 + 8 (l % 2))
  int lc, row0;   // for the clamped last chunk
};

// Part 0 (K), 1 (Q) or 2 (V, wave 3 only) of the tiles of chunk c into a tile ring slot, with
// one KiB of the chunk's T' fragments (tp: its record): 5, 5 and 1 (+ kDmaV) instructions.  kb,
// qb and vb point at row 0 of this workgroup's head in bytes; rows past the sequence end are
// clamped to its last row, which the compute waves never use.
template <int Part>
__device__ __forceinline__ void dma_tiles(int c, int tb, int te, int Hk, int Hv, int pw, int l,
                                          const unsigned char *kb, const unsigned char *qb,
                                          const unsigned char *vb, const uint8_t *tp,
                                          const ProducerLanes &pl, unsigned slot) {
  const int t0 = tb + kChunk * c;
  const int L = min(kChunk, te - t0);
  const size_t rs = (size_t)Hk * kDim * 2, vrs = (size_t)Hv * kDim * 2;
  // T' KiB pw + 4 Part of this chunk's record
  dma16s(tp + (pw + 4 * Part) * 1024, 16 * l, slot + kTT + (pw + 4 * Part) * 1024);
  if (Part < 2) {
    const unsigned char *base = (Part == 0 ? kb : qb) + (size_t)t0 * rs;
    const unsigned dst = slot + (Part == 0 ? kTK : kTQ);
    if (L == kChunk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16s(base + 16 * i * rs, pl.tile, dst + (4 * i + pw) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t off = (uint32_t)min(pl.row0 + 16 * i, L - 1) * (uint32_t)rs + 16 * pl.lc;
        dma16s(base, off, dst + (4 * i + pw) * 1024);
      }
    }
  } else if (pw == 3) {
    const unsigned char *vc = vb + (size_t)t0 * vrs;
#pragma unroll
    for (int m = 0; m < kDmaV; ++m) {
      if (L == kChunk) {
        dma16s(vc + 32 * m * vrs, pl.v, slot + kTV + m * 1024);
      } else {
        const uint32_t off = (uint32_t)min(32 * m + (l >> 1), L - 1) * (uint32_t)vrs + (pl.v % (uint32_t)vrs);
        dma16s(vc, off, slot + kTV + m * 1024);
      }
    }
  }
}
__device__ __forceinline__ void dma_tiles_all(int c, int tb, int te, int Hk, int Hv, int pw, int l,
                                              const unsigned char *kb, const unsigned char *qb,
                                              const unsigned char *vb, const uint8_t *tp,
                                              const ProducerLanes &pl, unsigned slot) {
  dma_tiles<0>(c, tb, te, Hk, Hv, pw, l, kb, qb, vb, tp, pl, slot);
  dma_tiles<1>(c, tb, te, Hk, Hv, pw, l, kb, qb, vb, tp, pl, slot);
  dma_tiles<2>(c, tb, te, Hk, Hv, pw, l, kb, qb, vb, tp, pl, slot);
}

// The record of a chunk (chunk_prep.hip).  Its T' fragments (12 KiB) travel with the tiles, two
// chunks ahead.  Its P fragments (6 KiB) are each read by exactly one output wave (row block w's
// by output wave w), so they go from global memory (L2, warmed by the prefetch wave) straight into
// that wave's registers with 16-byte loads, 1 KiB contiguous per fragment, issued one chunk ahead
// right after the previous fragments' last use.  Row block w owns fragments frag_base(w) and, for
// w >= 2, frag_base(w) + 1; waves 0 and 1 load fragment frag_base(w) twice so that every wave
// issues the same loads.  The decays (512 B, read by all eight waves) go to a small LDS ring.
__device__ __forceinline__ const uint8_t *rec_at(const uint8_t *rec, int64_t slot, int h, int Hv) {
  return rec + ((size_t)slot * Hv + h) * kRecBytes;
}
__device__ __forceinline__ int frag_base(int w) { return w < 2 ? w : 2 * w - 2; }
__device__ __forceinline__ int frag_next(int w) { return w < 2 ? w : 2 * w - 1; }

struct PFrags {
  bf16x8 p[2];  // P fragments frag_base(w), frag_next(w)
};
__device__ __forceinline__ void load_p(PFrags &r, const uint8_t *rp, int w, int l) {
  r.p[0] = *reinterpret_cast<const bf16x8 *>(rp + kRecP + frag_base(w) * kFragBytes + l * 16);
  r.p[1] = *reinterpret_cast<const bf16x8 *>(rp + kRecP + frag_next(w) * kFragBytes + l * 16);
}
// Decays of chunk slot `slot_idx` into a decay ring slot: lanes 0..31, 16 bytes each.
__device__ __forceinline__ void dma_dec(int64_t slot_idx, int h, int Hv, int l, const uint8_t *rec,
                                        unsigned slot) {
  if (l < kDecBytes / 16) dma16s(rec_at(rec, slot_idx, h, Hv) + kRecEG, 16 * l, slot);
}
// Offsets in a decay ring slot.
constexpr int kDecEG = 0;
constexpr int kDecED = kRecED - kRecEG;

// L2 warm-up: one 4-byte load per 128-byte line.  The lines that the producers of all
// workgroups sharing them will load -- the K and Q tiles (shared by the r = Hv / Hk heads of a
// k-head and their 8 column slices), the v-head's record and V rows (shared by its 8 slices) --
// are dealt out to those workgroups, so that each line is pulled once per L2.  gi is this
// workgroup's index among the ng = 8 r sharing the k-head.  Lane slot s = 64 j + l of touch
// instruction j names one line of chunk 0 (ptr) and the distance to the same line of the next
// chunk (adv); inactive slots have ptr = nullptr.
struct PrefetchLane {
  const unsigned char *ptr[2];
  uint32_t adv[2];
  int row[2];  // the line's token row within a chunk; -1 for record lines (no rows)
};
__device__ __forceinline__ PrefetchLane prefetch_lanes(int tb, int64_t slot0, int hk, int h, int Hk,
                                                       int Hv, int tile, int gi, int ng, int l,
                                                       const unsigned short *q,
                                                       const unsigned short *k,
                                                       const unsigned short *v,
                                                       const uint8_t *rec) {
  PrefetchLane pf;
  const int nkq = 4 * kChunk / ng;                   // K and Q lines: 64 rows x 2 lines each
  const int nrec = (kRecBytes / 128 - tile + 7) / 8;  // record lines tile, tile + 8, ...
  constexpr int nv = 2 * kChunk / kDvTiles;           // V lines: 64 rows x 2 lines (256 B a row)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int s = 64 * j + l;
    pf.ptr[j] = nullptr;
    pf.adv[j] = 0;
    pf.row[j] = -1;
    if (s < nkq) {
      const int m = gi + ng * s;
      const unsigned short *base = (m >> 7) ? q : k;
      pf.ptr[j] = reinterpret_cast<const unsigned char *>(
                      base + ((size_t)(tb + ((m >> 1) & 63)) * Hk + hk) * kDim) + 128 * (m & 1);
      pf.adv[j] = (uint32_t)(kChunk * Hk * kDim * 2);
      pf.row[j] = (m >> 1) & 63;
    } else if ((s -= nkq) < nrec) {
      pf.ptr[j] = rec + ((size_t)slot0 * Hv + h) * kRecBytes + 128 * (tile + 8 * s);
      pf.adv[j] = (uint32_t)(Hv * kRecBytes);
    } else if ((s -= nrec) < nv) {
      const int m = tile + kDvTiles * s;
      pf.ptr[j] = reinterpret_cast<const unsigned char *>(
                      v + ((size_t)(tb + (m >> 1)) * Hv + h) * kDim) + 128 * (m & 1);
      pf.adv[j] = (uint32_t)(kChunk * Hv * kDim * 2);
      pf.row[j] = m >> 1;
    }
  }
  return pf;
}

// Output rows 16 pw .. 16 pw + 15 of chunk c, left by output wave pw in its staging slot (rows
// 4 g .. 4 g + 3 of column j at byte 8 (16 g + j)), to global memory.  One transposing read gives
// lane i of lane group g row 4 g + i % 4, columns 4 (i / 4) .. + 3: lane r of the group names
// column 4 (r % 4) + r / 4, rows 4 g .. 4 g + 3 (see lds_read_tr16).  ob points at column d0 of
// this head in row 0 (bytes); ooff = row * Hv * 256 + 8 (i / 4) is the lane's fixed offset.
// nt: streaming (non-temporal) stores, chosen by the host when all of o fits in L2 -- then the
// dirty o lines would otherwise be written back at the kernel's end, after the last chunk; a
// larger o is mostly evicted during the kernel anyway, and its 32-byte column slices merge into
// whole lines in L2 first.  When the next kernel reads o (the mixer's gated RMSNorm), cached
// stores keep it in L2 for that kernel whatever its size.
template <bool kNt>
__device__ __forceinline__ void store_o(int c, int tb, int te, int Hv, int pw, int l,
                                        const unsigned char *slot, unsigned char *ob, uint32_t ooff) {
  const int g = l >> 4, i = l & 15;
  const int col = 4 * (i & 3) + (i >> 2);
  const v4i16 val = lds_read_tr16(slot + 8 * (16 * g + col));
  const int t0 = tb + kChunk * c;
  if (16 * pw + 4 * g + (i & 3) < min(kChunk, te - t0)) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 *dst = reinterpret_cast<u32x2 *>(ob + (size_t)t0 * Hv * kDim * 2 + ooff);
    if (kNt) __builtin_nontemporal_store(__builtin_bit_cast(u32x2, val), dst);
    else *dst = __builtin_bit_cast(u32x2, val);
  }
}

// ---- The gated RMSNorm fused into the output path (mixer; see NormOut) ------------------------
// The rows leave the output waves in store_o's layout: lane i of lane group g holds row
// 16 pw + 4 g + i % 4 of the chunk, columns 4 (i / 4) .. + 3 of the workgroup's 16, as bf16 -- the
// rule's output at its rounding point.  Per chunk an output wave (norm_step) publishes its rows'
// sums of squares over those 16 columns, issues the loads of the eight tile sums of the previous
// chunk's rows, and finishes the chunk before that: waits, if it must, until all eight tile sums of
// its rows are written, and stores y for its own 16 columns.  The other workgroups of the head walk
// the same chunks at the same pace, so their sums are written about two chunks before they are
// needed; the wait is bounded (kNormSpin) and only terminates early because the kernel is launched
// cooperatively: every workgroup of the head is resident and progresses.  o never leaves the
// workgroup, and the separate norm kernel's pass over o and z disappears.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kNormSpin = 1 << 22;  // sleeps of ~64 clocks: far beyond any in-order progress
struct NormRow {
  v4i16 o;   // bf16 o of the lane's row, 4 columns
  u32x2 z;   // bf16 z of the same
  int t;     // the row's token, -1 past the sequence end
  int tl;    // a token of the same chunk that exists (t, or the chunk's first)
};
struct NormSums {
  uint32_t a, b;  // tile sums 2 (i / 4) and 2 (i / 4) + 1 of the lane's row
};
__device__ __forceinline__ NormSums norm_load(const NormOut &no, const NormRow &r, int Hv, int h, int l) {
  const uint32_t *p = no.part + ((size_t)r.tl * Hv + h) * kDvTiles + 2 * ((l & 15) >> 2);
  return NormSums{__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                  __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
}
// The row slice of chunk c staged by out_stage: publish its tile sum of squares, load its z.
__device__ __forceinline__ NormRow norm_stage(int c, int tb, int te, int Hv, int h, int d0, int tile, int pw,
                                              int l, const unsigned char *slot, const NormOut &no) {
  const int g = l >> 4, i = l & 15;
  NormRow r;
  r.o = lds_read_tr16(slot + 8 * (16 * g + 4 * (i & 3) + (i >> 2)));
  const int t0 = tb + kChunk * c, row = 16 * pw + 4 * g + (i & 3);
  r.t = row < min(kChunk, te - t0) ? t0 + row : -1;
  r.tl = r.t >= 0 ? r.t : t0;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = bits_to_float((unsigned short)r.o[e]);
    ss += x * x;
  }
  ss += __shfl_xor(ss, 4, 64);  // the row's four lanes: i, i ^ 4, i ^ 8, i ^ 12
  ss += __shfl_xor(ss, 8, 64);
  uint32_t bits = __float_as_uint(ss);
  if (bits == kPartEmpty) bits = 0x7fc00000u;  // a NaN sum must not read as "not yet written"
  if (r.t >= 0 && (i >> 2) == 0)
    __hip_atomic_store(no.part + ((size_t)r.t * Hv + h) * kDvTiles + tile, bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  r.z = *reinterpret_cast<const u32x2 *>(no.z + ((size_t)r.tl * Hv + h) * kDim + d0 + 4 * (i >> 2));
  return r;
}
// y of a staged row slice from the eight tile sums of its row (loaded as sm).
template <bool kNt>
__device__ __forceinline__ void norm_finish(const NormRow &r, NormSums sm, u32x2 wv, int Hv, int h, int d0,
                                            int l, const NormOut &no) {
  bool empty = sm.a == kPartEmpty || sm.b == kPartEmpty;
  for (int it = 0; __any(empty) && it < kNormSpin; ++it) {
    __builtin_amdgcn_s_sleep(1);
    sm = norm_load(no, r, Hv, h, l);
    empty = sm.a == kPartEmpty || sm.b == kPartEmpty;
  }
  float ss = __uint_as_float(sm.a) + __uint_as_float(sm.b);
  ss += __shfl_xor(ss, 4, 64);
  ss += __shfl_xor(ss, 8, 64);
  const float rn = rsqrt_hw(ss * (1.f / kDim) + no.eps);
  float yv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const unsigned short zb = (unsigned short)(r.z[e >> 1] >> (16 * (e & 1)));
    const unsigned short wb = (unsigned short)(wv[e >> 1] >> (16 * (e & 1)));
    yv[e] = bits_to_float((unsigned short)r.o[e]) * rn * bits_to_float(wb) * silu(bits_to_float(zb));
  }
  if (r.t >= 0) {
    u32x2 *dst = reinterpret_cast<u32x2 *>(no.y + ((size_t)r.t * Hv + h) * kDim + d0 + 4 * ((l & 15) >> 2));
    const u32x2 val = {pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])};
    if (kNt) __builtin_nontemporal_store(val, dst);
    else *dst = val;
  }
}

// The output path o = e^G o (Q H) + P U~ for row block w of a chunk, on the output wave that
// shares a SIMD with compute wave w.  It issues no global->LDS loads: a wave's LDS reads wait for
// its own global->LDS loads still in flight, which would tie these reads to load latency.  out_qh
// runs between b1 and b2: Q H needs the chunk's entry state, which the compute waves overwrite in
// phase 3, and the Q tile's slot is not refilled before chunk c + 1.  out_stage runs once U~ is in
// LDS (after b2; the compute waves rewrite U~ only after b1 of the next chunk, so one buffer
// serves): it adds P U~ and stages the rows in this wave's LDS slot (lane-linear: rows 4 lg .. + 3
// of column lj at byte 8 l); they are read back transposed and stored between b1 and b2 of the
// next chunk (store_o).
__device__ __forceinline__ f32x4 out_qh(const unsigned char *qt, const unsigned char *Ht, int w, int l) {
  const int lj = l & 15, lg = l >> 4;
  f32x4 O = zero4();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    O = mfma_bf16(lds_bf16x8(qt + swz(16 * w + lj, 32 * ks + 8 * lg)),
                  lds_bf16x8(Ht + vmaj(lj, 32 * ks + 8 * lg)), O);
  return O;
}
// The LDS operands of out_stage for row block w: e^G of its rows and the B operands of P U~.
struct OutOps {
  f32x4 eg;
  bf16x8 u[2];
};
__device__ __forceinline__ OutOps out_fetch(const unsigned char *ds, const unsigned char *Uo, int w, int l) {
  const int lj = l & 15, lg = l >> 4;
  OutOps r;
  r.eg = *reinterpret_cast<const f32x4 *>(ds + kDecEG + (16 * w + 4 * lg) * 4);
  r.u[0] = lds_bf16x8(Uo + pmaj(lj, 4 * lg));
  r.u[1] = w >= 2 ? lds_bf16x8(Uo + pmaj(lj, 32 + 4 * lg)) : r.u[0];
  return r;
}
__device__ __forceinline__ void out_stage(f32x4 O, const PFrags &r, const OutOps &x, int w, int l,
                                          unsigned char *oslot) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) O[rr] *= x.eg[rr];
  O = mfma_bf16(r.p[0], x.u[0], O);
  if (w >= 2) O = mfma_bf16(r.p[1], x.u[1], O);
  store_u32x2(oslot + 8 * l, pack_bf16x2(O[0], O[1]), pack_bf16x2(O[2], O[3]));
}

// Compute wave w's K rows 16 w .. 16 w + 15 of the tile in ring slot ts, as the A operands of
// X = K H: ka[ks][p] holds keys 32 ks + 64 p + 8 lg .. + 7 in lane group lg.
__device__ __forceinline__ void read_k_rows(bf16x8 (&ka)[2][2], const unsigned char *ts, int w, int l) {
  const int lj = l & 15, lg = l >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int p = 0; p < 2; ++p) ka[ks][p] = lds_bf16x8(ts + kTK + swz(16 * w + lj, 32 * ks + 64 * p + 8 * lg));
}

// This wave's state slice into the H exchange buffers as bf16 hi (Ht) and lo (Htl = bf16(H - hi)):
// the B operands of X = K H (hi and lo) and Q H (hi only) in the next chunk.
__device__ __forceinline__ void write_ht(unsigned char *Ht, unsigned char *Htl, const f32x4 (&H)[2],
                                         int w, int l) {
  const int lj = l & 15, lg = l >> 4;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    uint32_t h0, l0, h1, l1;
    split_pair(H[a][0], H[a][1], h0, l0);
    split_pair(H[a][2], H[a][3], h1, l1);
    const int off = vmaj(lj, state_key(w, a, 4 * lg));
    store_u32x2(Ht + off, h0, h1);
    store_u32x2(Htl + off, l0, l1);
  }
}

// One chunk on compute wave w: tile ring slot ts (K, Q, V tiles and T' fragments), decay ring
// slot ds.  ka holds this wave's K rows of the chunk (the A operands of X = K H), read during the
// previous step; once the step has read U~ it reads those of the next chunk from slot tsn (landed
// by b2, see the producers), so that phase 1 -- the step's LDS-heaviest -- reads only H, V and
// the decays.  Rows past the sequence end hold clamped data; they need no masking because T' has
// zero rows and columns there (beta = 0), so U~ is zero on them, and their output rows are never
// stored.  The output path runs on the output waves (out_qh, out_stage).  With kWriteHt the step
// ends with the bf16 copy of the new state in the exchange buffer and the chunk's last barrier (b3);
// without it the caller does both, after any change of H between items.
template <bool kWriteHt>
__device__ __forceinline__ void chunk_step(const unsigned char *ts, const unsigned char *tsn,
                                           const unsigned char *ds, int w, int l, bf16x8 (&ka)[2][2],
                                           f32x4 (&H)[2], unsigned char *Ht,
                                           unsigned char *Htl, unsigned char *Rh, unsigned char *Rl,
                                           unsigned char *Uh, unsigned char *Ul, unsigned char *Uo,
                                           bool zero_v = false) {
  const int lj = l & 15, lg = l >> 4;
  const unsigned char *kt = ts + kTK;

  // X = K H (contraction over the 128 keys; B operands = H hi and lo from LDS), in two chains
  f32x4 X = zero4(), X2 = zero4();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    X = mfma_bf16(ka[ks][0], lds_bf16x8(Ht + vmaj(lj, 32 * ks + 8 * lg)), X);
    X2 = mfma_bf16(ka[ks][1], lds_bf16x8(Ht + vmaj(lj, 32 * ks + 64 + 8 * lg)), X2);
    X = mfma_bf16(ka[ks][0], lds_bf16x8(Htl + vmaj(lj, 32 * ks + 8 * lg)), X);
    X2 = mfma_bf16(ka[ks][1], lds_bf16x8(Htl + vmaj(lj, 32 * ks + 64 + 8 * lg)), X2);
  }
  X += X2;
  const f32x4 eg = *reinterpret_cast<const f32x4 *>(ds + kDecEG + (16 * w + 4 * lg) * 4);
  const f32x4 ed = *reinterpret_cast<const f32x4 *>(ds + kDecED + (16 * w + 4 * lg) * 4);
  const float egc = *reinterpret_cast<const float *>(ds + kDecEG + (kChunk - 1) * 4);
  // V[16 w + 4 lg + rr][lj], rr = 0..3, in one transposing read: lane r of each lane group names
  // row 16 w + 4 lg + r / 4, columns 4 (r % 4) .. + 3 of the row-major V tile.
  float vv[4];
  {
    const v4i16 v4 = lds_read_tr16(ts + kTV + ((16 * w + 4 * lg + (lj >> 2)) * kDvTile + 4 * (lj & 3)) * 2);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) vv[rr] = zero_v ? 0.f : bits_to_float((unsigned short)v4[rr]);
  }

  // R = V - e^G o X (hi/lo to LDS, value-major)
  {
    float R[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) R[rr] = vv[rr] - eg[rr] * X[rr];
    uint32_t h0, l0, h1, l1;
    split_pair(R[0], R[1], h0, l0);
    split_pair(R[2], R[3], h1, l1);
    store_u32x2(Rh + vmaj(lj, 16 * w + 4 * lg), h0, h1);
    store_u32x2(Rl + vmaj(lj, 16 * w + 4 * lg), l0, l1);
  }
  __syncthreads();

  // U~ = T' R for row block w (3 hi/lo terms; row blocks 2, 3 need two token steps); the K^T
  // fragments of phase 3 are read here, behind the T' and R reads.
  bf16x8 kc[2][2];
  f32x4 U = zero4();
  {
    const unsigned char *tt = ts + kTT + frag_base(w) * kFragBytes + l * 16;
    const bf16x8 th = lds_bf16x8(tt), tl = lds_bf16x8(tt + kTpBytes / 2);
    const bf16x8 bh = lds_bf16x8(Rh + vmaj(lj, 8 * lg));
    const bf16x8 bl = lds_bf16x8(Rl + vmaj(lj, 8 * lg));
    // K^T fragments for the state update, read transposed from the K tile: fragment (accumulator
    // a, token step ks), lane (lj, lg) holds K[token 32 ks + 8 lg + e][state_key(w, a, lj)].
    // ds_read_b64_tr_b16: within each 16-lane group, lane r names 4 consecutive bf16 (row r of a
    // 16 x 4 matrix M) and lane i receives M[4 j + i / 4][i % 4], j = 0..3.  With lane r = 4 j + q
    // naming K[token t + j][state_key(w, a, 4 q) .. + 3], lane i receives K[t .. t + 3] of key
    // state_key(w, a, i): half a fragment (4 tokens) per read.
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int key = state_key(w, a, 4 * (lj & 3));
        const int tok = 32 * ks + 8 * lg + (lj >> 2);
        const v4i16 lo4 = lds_read_tr16(kt + swz(tok, key));
        const v4i16 hi4 = lds_read_tr16(kt + swz(tok + 4, key));
        kc[a][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    U = mfma_bf16(th, bh, U);
    U = mfma_bf16(th, bl, U);
    U = mfma_bf16(tl, bh, U);
    if (w >= 2) {
      const bf16x8 th1 = lds_bf16x8(tt + kFragBytes), tl1 = lds_bf16x8(tt + kFragBytes + kTpBytes / 2);
      const bf16x8 bh1 = lds_bf16x8(Rh + vmaj(lj, 32 + 8 * lg));
      const bf16x8 bl1 = lds_bf16x8(Rl + vmaj(lj, 32 + 8 * lg));
      U = mfma_bf16(th1, bh1, U);
      U = mfma_bf16(th1, bl1, U);
      U = mfma_bf16(tl1, bh1, U);
    }
  }
  {
    uint32_t h0, l0, h1, l1;
    split_pair(ed[0] * U[0], ed[1] * U[1], h0, l0);
    split_pair(ed[2] * U[2], ed[3] * U[3], h1, l1);
    store_u32x2(Uh + vmaj(lj, 16 * w + 4 * lg), h0, h1);
    store_u32x2(Ul + vmaj(lj, 16 * w + 4 * lg), l0, l1);
    store_u32x2(Uo + pmaj(lj, 16 * w + 4 * lg), pack_bf16x2(U[0], U[1]), pack_bf16x2(U[2], U[3]));
  }
  __syncthreads();

  // H = e^{G_last} H + K^T (e^{G_last - G} o U~)  (decayed U~ hi + lo); the next chunk's K rows
  // are read behind U~.
  bf16x8 bh[2], bl[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bh[ks] = lds_bf16x8(Uh + vmaj(lj, 32 * ks + 8 * lg));
    bl[ks] = lds_bf16x8(Ul + vmaj(lj, 32 * ks + 8 * lg));
  }
  read_k_rows(ka, tsn, w, l);
#pragma unroll
  for (int a = 0; a < 2; ++a) H[a] *= egc;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      H[a] = mfma_bf16(kc[a][ks], bh[ks], H[a]);
      H[a] = mfma_bf16(kc[a][ks], bl[ks], H[a]);
    }
  }
  if constexpr (kWriteHt) {
    write_ht(Ht, Htl, H, w, l);
    __syncthreads();  // b3
  }
}

// ---- Work items --------------------------------------------------------------------------------
// An item is (sequence n, v-head h, 16-column tile).  The grid has G <= one workgroup per CU
// (G a multiple of 8); workgroup b takes the items of rounds k = 0, 1, ...: item
// lid = k G + (b % 8) (G / 8) + b / 8, as long as lid < N Hv 8.  Workgroup b runs on XCD b % 8,
// so within a round each XCD holds a contiguous range of items -- the 16 workgroups of a k-head
// (two v-heads x 8 tiles) share an L2 -- and a workgroup keeps one tile in every round.  A
// workgroup walks the chunks of its items as one stream of steps, so the loads of the next item
// overlap the last chunks of the current one.
struct Item {
  int n, h, hk, tb, te, nc;
  int64_t slot0;  // record slot of chunk 0: tb / 64 + n
};
struct Walker {
  int k, c;  // item round, chunk within the item
  int ord;   // ordinal of the item among the workgroup's non-empty items (the end: one past them)
  Item it;
  bool valid;
};
struct Grid {
  int G, total, Hv, r;  // r = Hv / Hk
};
__device__ __forceinline__ bool item_at(const Grid &g, int k, const int32_t *cu, Item &it) {
  const int b = blockIdx.x;
  const int64_t lid = (int64_t)k * g.G + (b % 8) * (g.G / 8) + b / 8;
  if (lid >= g.total) return false;
  const int rest = (int)(lid / kDvTiles);
  it.h = rest % g.Hv;
  it.n = rest / g.Hv;
  it.hk = it.h / g.r;
  it.tb = cu[it.n];
  it.te = cu[it.n + 1];
  it.nc = (it.te - it.tb + kChunk - 1) / kChunk;
  it.slot0 = it.tb / kChunk + it.n;
  return true;
}
// The next item with at least one chunk after round W.k; W.valid = false past the last.
__device__ __forceinline__ void next_item(Walker &W, const Grid &g, const int32_t *cu) {
  ++W.ord;
  for (;;) {
    ++W.k;
    if (!item_at(g, W.k, cu, W.it)) {
      W.valid = false;
      return;
    }
    if (W.it.nc > 0) {
      W.c = 0;
      W.valid = true;
      return;
    }
  }
}
__device__ __forceinline__ Walker first_step(const Grid &g, const int32_t *cu) {
  Walker W;
  W.k = -1;
  W.ord = -1;
  next_item(W, g, cu);
  return W;
}
__device__ __forceinline__ void next_step(Walker &W, const Grid &g, const int32_t *cu) {
  if (++W.c == W.it.nc) next_item(W, g, cu);
}
// Look-ahead for loads: past the last step it stays on the last step (a reload into a slot that is
// no longer read), so that every step issues the same loads.
__device__ __forceinline__ void next_step_clamped(Walker &W, const Grid &g, const int32_t *cu) {
  Walker t = W;
  next_step(t, g, cu);
  if (t.valid) W = t;
}

// Item ring.  The prefetch wave, whose walker runs kPrefetchAhead - 1 steps ahead, publishes each
// item it enters (and, past the last, an end marker) in LDS slot ord % kRingItems; the other waves
// take their items from there inside the loop.  Their own walk would load cu (and h0_index) with
// scalar loads at every change of item, and those loads sat on the chain (measured on 7 sequences
// of about 97 tokens: an item's first and last chunk steps took 1.4x and 1.3x a middle one).  A
// slot is rewritten kRingItems items after it was written, when every wave has moved past its item.
// Slot: k, n, h, hk, tb, te, nc, and the row of the initial-state pool the item starts from
// (-1: zeros).
constexpr int kRingItems = 8;
constexpr int kRingWords = 8;
// During step s the prefetch wave writes items up to cur + kPrefetchAhead (cur: the item of step
// s), into the slot of the item kRingItems before, while the other waves still read items from cur
// on: that earlier item must be older than cur.
static_assert(kRingItems > kPrefetchAhead, "a ring slot would be rewritten while still read");
__device__ __forceinline__ int h0_row(int n, const float *h0, const int32_t *h0_index, int num_h0) {
  if (!h0) return -1;
  const int r = h0_index ? h0_index[n] : n;
  return r >= 0 && r < num_h0 ? r : -1;
}
// Writes W's item (or the end marker) into its slot; lane 0 stores.  The caller waits for the
// store (lgkmcnt) before the barrier after which other waves read the slot.
__device__ __forceinline__ void ring_publish(int *ring, const Walker &W, const float *h0,
                                             const int32_t *h0_index, int num_h0, int l) {
  int4 a, b;
  a.x = W.k;
  if (W.valid) {
    a.y = W.it.n;
    a.z = W.it.h;
    a.w = W.it.hk;
    b.x = W.it.tb;
    b.y = W.it.te;
    b.z = W.it.nc;
    b.w = h0_row(W.it.n, h0, h0_index, num_h0);
  } else {
    a.y = -1;
    a.z = a.w = b.x = b.y = b.z = b.w = 0;
  }
  if (l == 0) {
    int4 *p = reinterpret_cast<int4 *>(ring + kRingWords * (W.ord % kRingItems));
    p[0] = a;
    p[1] = b;
  }
}
// Item ord from the ring (chunk 0); h0r: its initial-state row.
__device__ __forceinline__ void ring_item(Walker &W, int &h0r, const int *ring, int ord) {
  const int4 *p = reinterpret_cast<const int4 *>(ring + kRingWords * (ord % kRingItems));
  const int4 a = p[0], b = p[1];
  W.ord = ord;
  W.c = 0;
  W.k = __builtin_amdgcn_readfirstlane(a.x);
  W.it.n = __builtin_amdgcn_readfirstlane(a.y);
  W.it.h = __builtin_amdgcn_readfirstlane(a.z);
  W.it.hk = __builtin_amdgcn_readfirstlane(a.w);
  W.it.tb = __builtin_amdgcn_readfirstlane(b.x);
  W.it.te = __builtin_amdgcn_readfirstlane(b.y);
  W.it.nc = __builtin_amdgcn_readfirstlane(b.z);
  h0r = __builtin_amdgcn_readfirstlane(b.w);
  W.it.slot0 = W.it.tb / kChunk + W.it.n;
  W.valid = W.it.n >= 0;
}
__device__ __forceinline__ void next_step_ring(Walker &W, const int *ring) {
  if (++W.c == W.it.nc) {
    int h0r;
    ring_item(W, h0r, ring, W.ord + 1);
  }
}
__device__ __forceinline__ void next_step_ring_clamped(Walker &W, const int *ring) {
  Walker t = W;
  next_step_ring(t, ring);
  if (t.valid) W = t;
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Initial state slice of item it for compute wave w (H[a][rr] = state row state_key(w, a,
// 4 lg + rr), column d0 + lj): h0[h0_index[n]] of the pool, zeros outside [0, num_h0), h0[n]
// without an index, zeros without h0.
__device__ __forceinline__ void load_h0_row(f32x4 (&H)[2], int r, int h, const float *h0, int Hv,
                                            int d0, int w, int l) {
  const float *h0s = r >= 0 ? h0 + ((size_t)r * Hv + h) * kDim * kDim : nullptr;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = state_key(w, a, 4 * (l >> 4) + rr);
      H[a][rr] = h0s ? h0s[(size_t)key * kDim + d0 + (l & 15)] : 0.f;
    }
}
__device__ __forceinline__ void load_h0(f32x4 (&H)[2], const Item &it, const float *h0,
                                        const int32_t *h0_index, int num_h0, int Hv, int d0,
                                        int w, int l) {
  int r = -1;
  if (h0) {
    r = h0_index ? h0_index[it.n] : it.n;
    if (r < 0 || r >= num_h0) r = -1;
  }
  load_h0_row(H, r, it.h, h0, Hv, d0, w, l);
}
__device__ __forceinline__ void store_ht(const f32x4 (&H)[2], const Item &it, float *hT, int Hv,
                                         int d0, int w, int l) {
  if (!hT) return;
  // a uniform base and 32-bit lane offsets that do not change from item to item
  unsigned char *base = reinterpret_cast<unsigned char *>(hT + ((size_t)it.n * Hv + it.h) * kDim * kDim);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const uint32_t off = 4u * (uint32_t)(state_key(w, a, 4 * (l >> 4) + rr) * kDim + d0 + (l & 15));
      __builtin_nontemporal_store(H[a][rr], reinterpret_cast<float *>(base + off));
    }
}
// The compute waves' walk to the next non-empty item: an empty sequence's final state is its
// initial state, copied here.
__device__ __forceinline__ void next_item_copying(Walker &W, const Grid &g, const int32_t *cu,
                                                  const float *h0, const int32_t *h0_index,
                                                  int num_h0, float *hT, int d0, int w, int l) {
  ++W.ord;
  for (;;) {
    ++W.k;
    if (!item_at(g, W.k, cu, W.it)) {
      W.valid = false;
      return;
    }
    if (W.it.nc > 0) {
      W.c = 0;
      W.valid = true;
      return;
    }
    f32x4 Hc[2];
    load_h0(Hc, W.it, h0, h0_index, num_h0, g.Hv, d0, w, l);
    store_ht(Hc, W.it, hT, g.Hv, d0, w, l);
  }
}

}  // namespace

// One item per workgroup (launches whose items all fit on the device at once).  kNorm: the
// mixer's gated RMSNorm fused into the output path (y instead of o; cooperative launch only).
template <bool kONt, bool kNorm>
__global__ __launch_bounds__(kThreads, 1) void state_pass_kernel(
    const unsigned short *__restrict__ q, const unsigned short *__restrict__ k,
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const float *h0, const int32_t *__restrict__ h0_index, int num_h0,
    unsigned short *__restrict__ o, float *hT,  // hT may equal h0 when h0_index is NULL
    const uint8_t *__restrict__ rec, int Hk, int Hv, int t_one, SplitPass sp, NormOut no) {
  __shared__ __attribute__((aligned(16))) unsigned char tiles[kTileStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char decs[kDecStages * kDecBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Ht[kHtBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Htl[kHtBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Rh[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Rl[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Uh[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Ul[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Uo[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ostage[kComputeWaves * kOBytes];
  __shared__ __attribute__((aligned(16))) unsigned int touch_sink[64];

  const int lid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tile = lid % kDvTiles;
  const int rest = lid / kDvTiles;
  const int h = rest % Hv, n = rest / Hv;
  const int hk = h / (Hv / Hk);
  const int d0 = kDvTile * tile;
  const int tid = threadIdx.x, l = tid & 63, lj = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // n is a sequence, or with a time split a segment of sequence 0 (m chunks from chunk m n on).
  // With one sequence its bounds are 0 and T (t_one), so no load of cu_seqlens precedes the first
  // tile loads: it would put one more dependent memory round trip before chunk 0 can arrive.
  int tb, te, slot0;
  if (t_one >= 0) {
    tb = sp.segs ? min(kChunk * sp.m * n, t_one) : 0;
    te = sp.segs ? min(tb + kChunk * sp.m, t_one) : t_one;
    slot0 = sp.segs ? sp.m * n : 0;
  } else if (sp.segs) {
    tb = min(cu[0] + kChunk * sp.m * n, cu[1]);
    te = min(tb + kChunk * sp.m, cu[1]);
    slot0 = cu[0] / kChunk + sp.m * n;
  } else {
    tb = cu[n];
    te = cu[n + 1];
    slot0 = tb / kChunk + n;
  }
  const int nc = (te - tb + kChunk - 1) / kChunk;
  const size_t state_base = ((size_t)n * Hv + h) * kDim * kDim;
  const bool write_o = !sp.segs || sp.mode == 2;

  if (w == kPrefetchWave) {
    // Prefetch wave: warms L2 kPrefetchAhead chunks ahead of use and never waits for its loads
    // inside the loop (so a slow line holds up nothing).  Barriers as the compute waves.  A
    // sequence's partial last chunk is not warmed (its rows past the end must not be read).
    if (nc > 0) {
      const unsigned sink = (unsigned)(uintptr_t)touch_sink;
      const int r = Hv / Hk;
      PrefetchLane pf = prefetch_lanes(tb, slot0, hk, h, Hk, Hv, tile, tile * r + h % r,
                                       kDvTiles * r, l, q, k, v, rec);
      const int nfull = (te - tb) / kChunk;  // chunks 0 .. nfull - 1 are full
      // pointers of chunk 2
#pragma unroll
      for (int j = 0; j < 2; ++j) pf.ptr[j] += 2 * (size_t)pf.adv[j];
      dma_barrier();
      for (int c = 0; c < nc; ++c) {
        // chunks 2 .. kPrefetchAhead - 1 at the first iteration, then chunk c + kPrefetchAhead
        const int cbeg = c == 0 ? 2 : c + kPrefetchAhead;
        const int cend = min(c + kPrefetchAhead, nfull - 1);
        for (int cc = cbeg; cc <= cend; ++cc) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (pf.ptr[j]) touch(pf.ptr[j], sink);
            pf.ptr[j] += pf.adv[j];
          }
        }
        dma_barrier();
        dma_barrier();
        dma_barrier();
      }
    }
    wait_vmcnt<0>();  // no LDS write may land after the workgroup ends
    return;
  }

  if (w >= kOutputWave0) {
    // Output waves: o = e^G o (Q H) + P U~ for row block ow.  Barriers as the compute waves.  Q H
    // of chunk c is taken between b1 and b2 (H(c) is rewritten in phase 3; the Q tile's slot is
    // refilled during chunk c + 1), P U~ of chunk c before b1 of chunk c + 1 (U~ is rewritten only
    // after that barrier), so that nothing of the output path holds b3; the rows are stored between
    // b1 and b2 of chunk c + 1.
    const int ow = w - kOutputWave0;
    if (nc > 0) {
      unsigned char *ob = reinterpret_cast<unsigned char *>(o + (size_t)h * kDim + d0);
      unsigned char *oslot = ostage + ow * kOBytes;
      const uint32_t ooff = (uint32_t)(16 * ow + 4 * (l >> 4) + (l & 3)) * (uint32_t)(Hv * kDim * 2) +
                            8 * ((l & 15) >> 2);
      PFrags pf;
      load_p(pf, rec_at(rec, slot0, h, Hv), ow, l);
      f32x4 O = zero4();
      // fused norm: row slices of the previous chunk (na) and the one before (nb), and the tile
      // sums of na's rows loaded one step before their use
      NormRow na{}, nb{};
      NormSums sb{};
      u32x2 wv{};
      if constexpr (kNorm) wv = *reinterpret_cast<const u32x2 *>(no.w + d0 + 4 * ((l & 15) >> 2));
      auto norm_step = [&](int cc) {  // chunk cc staged; cc - 1 loads its sums; cc - 2 finishes
        const NormRow nr = norm_stage(cc, tb, te, Hv, h, d0, tile, ow, l, oslot, no);
        const NormSums s_new = norm_load(no, na, Hv, h, l);
        if (cc >= 2) norm_finish<kONt>(nb, sb, wv, Hv, h, d0, l, no);
        nb = na;
        sb = s_new;
        na = nr;
      };
      OutOps oo;  // LDS operands of chunk c's P U~, read in phase 3 of chunk c (LDS is lightly used there)
      __syncthreads();
      for (int c = 0; c < nc; ++c) {
        if (c > 0) {
          out_stage(O, pf, oo, ow, l, oslot);
          load_p(pf, rec_at(rec, slot0 + c, h, Hv), ow, l);
        }
        __syncthreads();  // b1
        if constexpr (kNorm) {
          if (c > 0) norm_step(c - 1);
        } else {
          if (c > 0 && write_o) store_o<kONt>(c - 1, tb, te, Hv, ow, l, oslot, ob, ooff);
        }
        O = out_qh(tiles + (c % kTileStages) * kTileBytes + kTQ, Ht, ow, l);
        __syncthreads();  // b2
        oo = out_fetch(decs + (c % kDecStages) * kDecBytes, Uo, ow, l);
        __syncthreads();  // b3
      }
      out_stage(O, pf, oo, ow, l, oslot);
      if constexpr (kNorm) {
        norm_step(nc - 1);
        if (nc >= 2) norm_finish<kONt>(nb, sb, wv, Hv, h, d0, l, no);  // chunk nc - 2
        norm_finish<kONt>(na, norm_load(no, na, Hv, h, l), wv, Hv, h, d0, l, no);  // chunk nc - 1
      } else {
        if (write_o) store_o<kONt>(nc - 1, tb, te, Hv, ow, l, oslot, ob, ooff);
      }
    }
    return;
  }

  if (w >= kComputeWaves) {
    // Producer waves.  Barriers: one before the loop, three per chunk, as the compute waves.
    const int pw = w - kComputeWaves;
    if (nc > 0) {
      const unsigned tiles_lds = (unsigned)(uintptr_t)tiles;
      const unsigned decs_lds = (unsigned)(uintptr_t)decs;
      const unsigned char *kb = reinterpret_cast<const unsigned char *>(k + (size_t)hk * kDim);
      const unsigned char *qb = reinterpret_cast<const unsigned char *>(q + (size_t)hk * kDim);
      const unsigned char *vb = reinterpret_cast<const unsigned char *>(v + (size_t)h * kDim);
      ProducerLanes pl;
      pl.row0 = 4 * pw + (l >> 4);
      pl.lc = (l & 15) ^ (pl.row0 & 15);
      pl.tile = (uint32_t)pl.row0 * (uint32_t)(Hk * kDim * 2) + 16 * pl.lc;
      pl.v = (uint32_t)(l >> 1) * (uint32_t)(Hv * kDim * 2) + 2 * (d0 + 8 * (l & 1));
      const int c1 = min(1, nc - 1);
      dma_tiles_all(0, tb, te, Hk, Hv, pw, l, kb, qb, vb, rec_at(rec, slot0, h, Hv), pl, tiles_lds);
      if (pw == kDecWave) dma_dec(slot0, h, Hv, l, rec, decs_lds);
      dma_tiles_all(c1, tb, te, Hk, Hv, pw, l, kb, qb, vb, rec_at(rec, slot0 + c1, h, Hv), pl,
                    tiles_lds + kTileBytes);
      if (pw == kDecWave) dma_dec(slot0 + c1, h, Hv, l, rec, decs_lds + kDecBytes);
      // chunk 0 has landed: only chunk 1's loads may still be in flight
      if (pw == 3) wait_vmcnt<kChunkCount(3)>();
      else if (pw == kDecWave) wait_vmcnt<kChunkCount(kDecWave)>();
      else wait_vmcnt<kChunkCount(0)>();
      dma_barrier();
      for (int c = 0; c < nc; ++c) {
        // Chunk c + 2 is loaded during chunk c, spread over its three phases, into tile and decay
        // slots (c + 2) % 3, which held chunk c - 1 (clamped reloads of the last chunk only go to
        // slots that are no longer read): K before b1, Q before b2, V and the decays before b3.
        const int cn = min(c + 2, nc - 1);
        const unsigned tslot = tiles_lds + ((c + 2) % kTileStages) * kTileBytes;
        const uint8_t *tp = rec_at(rec, slot0 + cn, h, Hv);
        dma_tiles<0>(cn, tb, te, Hk, Hv, pw, l, kb, qb, vb, tp, pl, tslot);
        dma_barrier();  // b1
        dma_tiles<1>(cn, tb, te, Hk, Hv, pw, l, kb, qb, vb, tp, pl, tslot);
        // Chunk c + 1 (loaded during chunk c - 1) must have landed before b2, after which the
        // compute waves read its K tile: loads complete in issue order, so it is enough that at
        // most this iteration's loads so far are in flight.
        wait_vmcnt<kPartsBeforeB2>();
        dma_barrier();  // b2
        dma_tiles<2>(cn, tb, te, Hk, Hv, pw, l, kb, qb, vb, tp, pl, tslot);
        if (pw == kDecWave) dma_dec(slot0 + cn, h, Hv, l, rec, decs_lds + ((c + 2) % kDecStages) * kDecBytes);
        dma_barrier();  // b3
      }
    }
    wait_vmcnt<0>();  // no LDS write may land after the workgroup ends
    return;
  }

  // State slice: H[a][rr] = H[key state_key(w, a, 4 lg + rr)][value d0 + lj].  Sequence n starts
  // from initial state h0_index[n] of the pool (zeros outside [0, num_h0)), or from state n.
  const float *h0s = nullptr;
  if (sp.segs) {
    if (sp.mode == 2) h0s = sp.h_in + state_base;
  } else if (h0) {
    const int r = h0_index ? h0_index[n] : n;
    if (r >= 0 && r < num_h0) h0s = h0 + ((size_t)r * Hv + h) * kDim * kDim;
  }
  const bool ident = sp.segs && sp.mode == 1;
  f32x4 H[2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = state_key(w, a, 4 * lg + rr);
      H[a][rr] = h0s ? h0s[(size_t)key * kDim + d0 + lj] : (ident && key == d0 + lj ? 1.f : 0.f);
    }

  if (nc > 0) {
    write_ht(Ht, Htl, H, w, l);
    __syncthreads();
    bf16x8 ka[2][2];
    read_k_rows(ka, tiles, w, l);
    // Unrolled over twice the period of the ring slots (3), so every slot address is a
    // compile-time offset rather than per-chunk address arithmetic on the compute waves (a
    // three-chunk body keeps more values live across its steps and spills).
    static_assert(kTileStages == 3 && kDecStages == 3, "the unroll assumes 3-slot rings");
    for (int c0 = 0; c0 < nc; c0 += 6) {
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        if (c0 + u < nc)
          chunk_step<true>(tiles + (u % 3) * kTileBytes, tiles + ((u + 1) % 3) * kTileBytes,
                           decs + (u % 3) * kDecBytes, w, l, ka, H, Ht, Htl, Rh, Rl, Uh, Ul, Uo, ident);
      }
    }
  }

  float *hdst = hT ? hT + state_base : nullptr;
  if (sp.segs)
    hdst = sp.mode < 2 ? sp.h_out + state_base
                       : (n == sp.segs - 1 && hT ? hT + (size_t)h * kDim * kDim : nullptr);
  if (hdst) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = state_key(w, a, 4 * lg + rr);
        if (sp.segs && sp.mode < 2)
          hdst[(size_t)key * kDim + d0 + lj] = H[a][rr];  // read by the next kernel: keep it cached
        else
          __builtin_nontemporal_store(H[a][rr], hdst + (size_t)key * kDim + d0 + lj);
      }
  }
}

// Persistent workgroups walking several items each (launches with more items than fit at once).
template <bool kONt>
__global__ __launch_bounds__(kThreads, 1) void state_pass_multi_kernel(
    const unsigned short *__restrict__ q, const unsigned short *__restrict__ k,
    const unsigned short *__restrict__ v, const int32_t *__restrict__ cu,
    const float *h0, const int32_t *__restrict__ h0_index, int num_h0,
    unsigned short *__restrict__ o, float *hT,  // hT may equal h0 when h0_index is NULL
    const uint8_t *__restrict__ rec, int Hk, int Hv, int total_items) {
  __shared__ __attribute__((aligned(16))) unsigned char tiles[kTileStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char decs[kDecStages * kDecBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Ht[kHtBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Htl[kHtBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Rh[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Rl[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Uh[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Ul[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Uo[kXBytes];
  __shared__ __attribute__((aligned(16))) unsigned char ostage[kComputeWaves * kOBytes];
  __shared__ __attribute__((aligned(16))) unsigned int touch_sink[64];
  __shared__ __attribute__((aligned(16))) int ring[kRingItems * kRingWords];

  const Grid gr{(int)gridDim.x, total_items, Hv, Hv / Hk};
  const int tile = (int)(((blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8) % kDvTiles);  // every round
  const int d0 = kDvTile * tile;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r = Hv / Hk;

  if (w == kPrefetchWave) {
    // Prefetch wave: warms L2 kPrefetchAhead steps ahead of use and never waits for its loads
    // inside the loop (so a slow line holds up nothing).  Barriers as the compute waves.  Of a
    // sequence's partial last chunk only the rows that exist are warmed (items of short sequences
    // are mostly such chunks).  Its walker pf, the step warmed next, runs kPrefetchAhead - 1 steps
    // ahead and publishes every item it enters, and the end, in the ring.  The walk (scalar loads
    // of cu and h0_index at item changes) is done between b1 and b2, where this wave has nothing
    // else to do; before b1 it only issues the step's loads.
    Walker cur = first_step(gr, cu);
    if (cur.valid) {
      const unsigned sink = (unsigned)(uintptr_t)touch_sink;
      Walker pf = cur;
      PrefetchLane pl;  // lines of chunk 0 of pf's item
      auto enter = [&]() {  // pf has entered an item, or the end
        ring_publish(ring, pf, h0, h0_index, num_h0, l);
        if (pf.valid)
          pl = prefetch_lanes(pf.it.tb, pf.it.slot0, pf.it.hk, pf.it.h, Hk, Hv, tile,
                              tile * r + pf.it.h - pf.it.hk * r, kDvTiles * r, l, q, k, v, rec);
      };
      auto advance = [&]() {
        next_step(pf, gr, cu);
        if (!pf.valid || pf.c == 0) enter();
      };
      auto warm = [&]() {  // step pf's lines
        const int rows = min(kChunk, pf.it.te - pf.it.tb - kChunk * pf.c);  // rows of this chunk
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (pl.ptr[j] && pl.row[j] < rows) touch(pl.ptr[j] + (size_t)pf.c * pl.adv[j], sink);
      };
      // steps 0 .. 2 into the ring before the first barrier; steps 2 .. kPrefetchAhead - 2 warmed
      // and steps 3 .. kPrefetchAhead - 1 published before b1 of step 0
      enter();
      advance();
      if (pf.valid) advance();
      wait_lgkmcnt0();
      dma_barrier();
      for (int cnt = kPrefetchAhead - 3; cnt > 0 && pf.valid; --cnt) {
        warm();
        advance();
      }
      wait_lgkmcnt0();
      for (int s = 0; cur.valid; ++s) {
        // step s + kPrefetchAhead - 1 warmed before b1; step s + kPrefetchAhead entered after b1
        if (pf.valid) warm();
        dma_barrier();  // b1
        if (pf.valid) advance();
        wait_lgkmcnt0();
        dma_barrier();  // b2
        dma_barrier();  // b3
        next_step_ring(cur, ring);
      }
    }
    wait_vmcnt<0>();  // no LDS write may land after the workgroup ends
    return;
  }

  if (w >= kOutputWave0) {
    // Output waves: o = e^G o (Q H) + P U~ for row block ow.  Barriers as the compute waves.  Q H
    // of step s between b1 and b2, then P U~, the rows' store and the next step's P load between b2
    // and b3 (U~ of step s is in LDS from b2 on and is rewritten only after b1 of step s + 1).
    // Unlike in the single-round kernel, whose b3 they would hold up, that is faster here (7
    // sequences at T = 677: 33.0 -> 31.0 us per pass, interleaved on one box).
    const int ow = w - kOutputWave0;
    Walker cur = first_step(gr, cu);
    if (cur.valid) {
      unsigned char *oslot = ostage + ow * kOBytes;
      const uint32_t ooff = (uint32_t)(16 * ow + 4 * (l >> 4) + (l & 3)) * (uint32_t)(Hv * kDim * 2) +
                            8 * ((l & 15) >> 2);
      PFrags pf;
      load_p(pf, rec_at(rec, cur.it.slot0, cur.it.h, Hv), ow, l);
      __syncthreads();
      for (int s = 0; cur.valid; ++s) {
        __syncthreads();  // b1
        const f32x4 O = out_qh(tiles + (s % kTileStages) * kTileBytes + kTQ, Ht, ow, l);
        __syncthreads();  // b2
        out_stage(O, pf, out_fetch(decs + (s % kDecStages) * kDecBytes, Uo, ow, l), ow, l, oslot);
        const int c_ = cur.c, tb_ = cur.it.tb, te_ = cur.it.te, h_ = cur.it.h;
        next_step_ring(cur, ring);
        if (cur.valid) load_p(pf, rec_at(rec, cur.it.slot0 + cur.c, cur.it.h, Hv), ow, l);
        store_o<kONt>(c_, tb_, te_, Hv, ow, l, oslot, reinterpret_cast<unsigned char *>(o + (size_t)h_ * kDim + d0),
                      ooff);
        __syncthreads();  // b3
      }
    }
    return;
  }

  if (w >= kComputeWaves) {
    // Producer waves.  Barriers: one before the loop, three per step, as the compute waves.
    const int pw = w - kComputeWaves;
    Walker cur = first_step(gr, cu);
    if (cur.valid) {
      const unsigned tiles_lds = (unsigned)(uintptr_t)tiles;
      const unsigned decs_lds = (unsigned)(uintptr_t)decs;
      ProducerLanes pl;
      pl.row0 = 4 * pw + (l >> 4);
      pl.lc = (l & 15) ^ (pl.row0 & 15);
      pl.tile = (uint32_t)pl.row0 * (uint32_t)(Hk * kDim * 2) + 16 * pl.lc;
      pl.v = (uint32_t)(l >> 1) * (uint32_t)(Hv * kDim * 2) + 2 * (d0 + 8 * (l & 1));
      // K, Q and V bases (bytes, row 0) of a step's head
#define GDN_BASES(W)                                                                              \
  reinterpret_cast<const unsigned char *>(k + (size_t)(W).it.hk * kDim),                          \
      reinterpret_cast<const unsigned char *>(q + (size_t)(W).it.hk * kDim),                      \
      reinterpret_cast<const unsigned char *>(v + (size_t)(W).it.h * kDim)
      Walker ld = cur;  // step 0, then 1
      dma_tiles_all(ld.c, ld.it.tb, ld.it.te, Hk, Hv, pw, l, GDN_BASES(ld),
                    rec_at(rec, ld.it.slot0 + ld.c, ld.it.h, Hv), pl, tiles_lds);
      if (pw == kDecWave) dma_dec(ld.it.slot0 + ld.c, ld.it.h, Hv, l, rec, decs_lds);
      next_step_clamped(ld, gr, cu);
      dma_tiles_all(ld.c, ld.it.tb, ld.it.te, Hk, Hv, pw, l, GDN_BASES(ld),
                    rec_at(rec, ld.it.slot0 + ld.c, ld.it.h, Hv), pl, tiles_lds + kTileBytes);
      if (pw == kDecWave) dma_dec(ld.it.slot0 + ld.c, ld.it.h, Hv, l, rec, decs_lds + kDecBytes);
      // step 0 has landed: only step 1's loads may still be in flight
      if (pw == 3) wait_vmcnt<kChunkCount(3)>();
      else if (pw == kDecWave) wait_vmcnt<kChunkCount(kDecWave)>();
      else wait_vmcnt<kChunkCount(0)>();
      dma_barrier();
      for (int s = 0; cur.valid; ++s) {
        // Step s + 2 is loaded during step s, spread over its three phases, into tile and decay
        // slots (s + 2) % 3, which held step s - 1 (clamped reloads of the last step only go to
        // slots that are no longer read): K before b1, Q before b2, V and the decays before b3.
        next_step_ring_clamped(ld, ring);
        const unsigned tslot = tiles_lds + ((s + 2) % kTileStages) * kTileBytes;
        const uint8_t *tp = rec_at(rec, ld.it.slot0 + ld.c, ld.it.h, Hv);
        dma_tiles<0>(ld.c, ld.it.tb, ld.it.te, Hk, Hv, pw, l, GDN_BASES(ld), tp, pl, tslot);
        dma_barrier();  // b1
        dma_tiles<1>(ld.c, ld.it.tb, ld.it.te, Hk, Hv, pw, l, GDN_BASES(ld), tp, pl, tslot);
        // Step s + 1 (loaded during step s - 1) must have landed before b2, after which the
        // compute waves read its K tile: loads complete in issue order, so it is enough that at
        // most this iteration's loads so far are in flight.
        wait_vmcnt<kPartsBeforeB2>();
        dma_barrier();  // b2
        dma_tiles<2>(ld.c, ld.it.tb, ld.it.te, Hk, Hv, pw, l, GDN_BASES(ld), tp, pl, tslot);
        if (pw == kDecWave)
          dma_dec(ld.it.slot0 + ld.c, ld.it.h, Hv, l, rec, decs_lds + ((s + 2) % kDecStages) * kDecBytes);
        dma_barrier();  // b3
        next_step_ring(cur, ring);
      }
#undef GDN_BASES
    }
    wait_vmcnt<0>();  // no LDS write may land after the workgroup ends
    return;
  }

  // Compute waves.  State slice: H[a][rr] = H[key state_key(w, a, 4 lg + rr)][value d0 + lj].
  // At the last chunk of an item the final state is stored and the next item's initial state,
  // loaded kPrefetchAhead - 1 chunks earlier (or from the item's first chunk on: items of short
  // sequences last one or two chunks, less than a load from memory), takes its place before H (hi
  // and lo) goes to LDS.
  Walker cur;
  cur.k = -1;
  cur.ord = -1;
  next_item_copying(cur, gr, cu, h0, h0_index, num_h0, hT, d0, w, l);
  if (!cur.valid) return;
  f32x4 H[2], Hn[2];
  load_h0(H, cur.it, h0, h0_index, num_h0, Hv, d0, w, l);
  Walker nx = cur;  // the next item: the second by the walk, later ones from the ring
  next_item(nx, gr, cu);
  if (nx.valid) load_h0(Hn, nx.it, h0, h0_index, num_h0, Hv, d0, w, l);
  write_ht(Ht, Htl, H, w, l);
  __syncthreads();
  bf16x8 ka[2][2];
  read_k_rows(ka, tiles, w, l);
  // Hf: the final state of the last item, whose registers the stores read after they issue.  It
  // stays live over the loop, so that no register of it is rewritten (which would wait for the
  // stores, and so for every load issued after them) before the next item's end.
  f32x4 Hf[2] = {};
  for (int s = 0; cur.valid; ++s) {
    asm volatile("" ::"v"(Hf[0]), "v"(Hf[1]));
    const bool last = cur.c == cur.it.nc - 1;
    // The ring holds the next item from kPrefetchAhead - 1 steps before its first chunk on.
    if (cur.ord > 0 && cur.c == max(0, cur.it.nc - (kPrefetchAhead - 1))) {
      int h0r;
      ring_item(nx, h0r, ring, cur.ord + 1);
      if (nx.valid) load_h0_row(Hn, h0r, nx.it.h, h0, Hv, d0, w, l);
    }
    chunk_step<false>(tiles + (s % kTileStages) * kTileBytes, tiles + ((s + 1) % kTileStages) * kTileBytes,
                      decs + (s % kDecStages) * kDecBytes, w, l, ka, H, Ht, Htl, Rh, Rl, Uh, Ul, Uo);
    if (last) {
      // The next item's state goes to LDS before this one's final state is stored: a wait for its
      // loads placed after the stores would wait for the stores too.
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        Hf[a] = H[a];
        if (nx.valid) H[a] = Hn[a];
      }
      write_ht(Ht, Htl, H, w, l);
      __builtin_amdgcn_sched_barrier(0);
      store_ht(Hf, cur.it, hT, Hv, d0, w, l);
      // empty items between this one and the next: their final state is their initial one
      for (int kk = cur.k + 1; kk < nx.k; ++kk) {
        Item e;
        item_at(gr, kk, cu, e);
        f32x4 Hc[2];
        load_h0(Hc, e, h0, h0_index, num_h0, Hv, d0, w, l);
        store_ht(Hc, e, hT, Hv, d0, w, l);
      }
      cur = nx;
    } else {
      ++cur.c;
      write_ht(Ht, Htl, H, w, l);
    }
    __syncthreads();  // b3
  }
}

// Initial states of the segments of a time-split sequence: hs[0] is the sequence's own initial
// state (h0 row h0_index[0], or row 0, or zeros), and hs[s] = phi[s-1] hs[s-1] + bend[s-1] for
// s = 1 .. segs - 1 -- a segment maps its initial state H to phi H + bend (states key-major, so the
// transition multiplies from the left).  fp32 on the matrix cores (v_mfma_f32_16x16x4_f32, exact
// products).  One workgroup per (v-head, 16-column tile), 8 waves; wave wv makes output rows
// 16 wv .. 16 wv + 15, the previous state's tile stays in LDS.
constexpr int kScanThreads = 512;
__global__ __launch_bounds__(kScanThreads) void state_scan_kernel(
    const float *__restrict__ phi, const float *__restrict__ bend, const float *h0,
    const int32_t *__restrict__ h0_index, int num_h0, float *__restrict__ hs, int segs, int Hv) {
  // [key][column] of the previous segment's initial state; key k sits at row hp_row(k), which
  // rotates each aligned group of 4 keys by k / 4, so the four lane groups' reads of keys
  // 16 j + 4 lg + e fall on different banks.
  __shared__ float Hp[kDim * kDvTile];
  auto hp_row = [](int k) { return (k & ~3) | ((k + (k >> 2)) & 3); };
  const int tile = blockIdx.x % kDvTiles, h = blockIdx.x / kDvTiles, d0 = kDvTile * tile;
  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, lj = l & 15, lg = l >> 4;
  const size_t hb = (size_t)h * kDim * kDim, seg = (size_t)Hv * kDim * kDim;
  const float *h0s = nullptr;
  if (h0) {
    const int r = h0_index ? h0_index[0] : 0;
    if (r >= 0 && r < num_h0) h0s = h0 + ((size_t)r * Hv + h) * kDim * kDim;
  }
  for (int e = tid; e < kDim * kDvTile; e += kScanThreads) {
    const int key = e / kDvTile, col = e % kDvTile;
    const float x = h0s ? h0s[(size_t)key * kDim + d0 + col] : 0.f;
    Hp[hp_row(key) * kDvTile + col] = x;
    hs[hb + (size_t)key * kDim + d0 + col] = x;
  }
  __syncthreads();
  // Product p = 4 j + e takes contraction index k = 16 j + 4 lg + e in lane group lg: load j of a
  // lane is 16 bytes of its row, and the four lane groups' loads j cover 64 contiguous bytes of
  // each row, so one load instruction touches 16 cache lines instead of 64.  Two register sets alternate: step s + 2's
  // operands are loaded into the set step s has just used, before step s's results are stored
  // (one counter tracks loads and stores in order, so a load issued after a store would wait
  // for the store).  The 32 products run as two independent chains.
  auto load_step = [&](int s, f32x4 (&a4)[kDim / 16], f32x4 &b4) {
    const float *P = phi + (size_t)(s - 1) * seg + hb + (size_t)(16 * wv + lj) * kDim + 4 * lg;
    const float *B = bend + (size_t)(s - 1) * seg + hb;
#pragma unroll
    for (int i = 0; i < kDim / 16; ++i) a4[i] = *reinterpret_cast<const f32x4 *>(P + 16 * i);
#pragma unroll
    for (int r = 0; r < 4; ++r) b4[r] = B[(size_t)(16 * wv + 4 * lg + r) * kDim + d0 + lj];
  };
  auto step = [&](int s, f32x4 (&a4)[kDim / 16], f32x4 &b4) {
    float hv[kDim / 4];  // B operands, all read before the first product
#pragma unroll
    for (int i = 0; i < kDim / 4; ++i) hv[i] = Hp[hp_row(16 * (i >> 2) + 4 * lg + (i & 3)) * kDvTile + lj];
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc0 = b4, acc1 = zero4();
#pragma unroll
    for (int i = 0; i < kDim / 4; i += 2) {
      acc0 = mfma_f32(a4[i / 4][i % 4], hv[i], acc0);
      acc1 = mfma_f32(a4[i / 4][i % 4 + 1], hv[i + 1], acc1);
    }
    const f32x4 acc = acc0 + acc1;
    __syncthreads();  // every wave has read Hp
    if (s + 2 < segs) load_step(s + 2, a4, b4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 16 * wv + 4 * lg + r;
      Hp[hp_row(key) * kDvTile + lj] = acc[r];
      hs[(size_t)s * seg + hb + (size_t)key * kDim + d0 + lj] = acc[r];
    }
    __syncthreads();
  };
  f32x4 aA[kDim / 16], bA, aB[kDim / 16], bB;
  if (segs > 1) load_step(1, aA, bA);
  if (segs > 2) load_step(2, aB, bB);
  for (int s = 1; s < segs; s += 2) {
    step(s, aA, bA);
    if (s + 1 >= segs) break;
    step(s + 1, aB, bB);
  }
}

void launch_state_scan(const float *phi, const float *bend, const float *h0, const int32_t *h0_index,
                       int num_h0, float *hs, int segs, int Hv, hipStream_t stream) {
  hipLaunchKernelGGL(state_scan_kernel, dim3(Hv * kDvTiles), dim3(kScanThreads), 0, stream, phi, bend,
                     h0, h0_index, num_h0, hs, segs, Hv);
}

hipError_t launch_state_pass(const void *q, const void *k, const void *v, const int32_t *cu,
                             const float *h0, const int32_t *h0_index, int num_h0, void *o, float *hT,
                             const void *rec, int64_t T, int N, int Hk, int Hv, int max_groups,
                             hipStream_t stream, SplitPass sp, const NormOut *norm, bool o_read_next) {
  // Items: N Hv 8 (a multiple of 8).  One round when they fit on the device at one workgroup per
  // CU (max_groups, a multiple of 8), else max_groups persistent workgroups.
  const int total = (sp.segs ? sp.segs : N) * Hv * kDvTiles;
  const int G = total <= max_groups ? total : max_groups;
  const bool o_nt = !o_read_next && (uint64_t)T * (uint64_t)Hv * kDim * 2 <= kOStreamBytes;
  int t_one = N == 1 ? (int)T : -1;  // cu_seqlens = {0, T}
  const unsigned short *q16 = static_cast<const unsigned short *>(q);
  const unsigned short *k16 = static_cast<const unsigned short *>(k);
  const unsigned short *v16 = static_cast<const unsigned short *>(v);
  unsigned short *o16 = static_cast<unsigned short *>(o);
  const uint8_t *r8 = static_cast<const uint8_t *>(rec);
  if (norm) {
    // every workgroup of a head must be resident for the fused norm's waits to end: cooperative
    // launch (the host plans this only for a single round without a time split)
    if (G != total || sp.segs) return hipErrorInvalidValue;
    NormOut no = *norm;
    void *args[] = {&q16, &k16, &v16, (void *)&cu, (void *)&h0, (void *)&h0_index, &num_h0, &o16, &hT,
                    &r8, &Hk, &Hv, &t_one, &sp, &no};
    const void *fn = o_nt ? reinterpret_cast<const void *>(&state_pass_kernel<true, true>)
                          : reinterpret_cast<const void *>(&state_pass_kernel<false, true>);
    return hipLaunchCooperativeKernel(fn, dim3(G), dim3(kThreads), args, 0, stream);
  }
  const NormOut none{};
  if (G == total)
    hipLaunchKernelGGL((o_nt ? state_pass_kernel<true, false> : state_pass_kernel<false, false>), dim3(G),
                       dim3(kThreads), 0, stream, q16, k16, v16, cu, h0, h0_index, num_h0, o16, hT,
                       r8, Hk, Hv, t_one, sp, none);
  else
    hipLaunchKernelGGL(o_nt ? state_pass_multi_kernel<true> : state_pass_multi_kernel<false>,
                       dim3(G), dim3(kThreads), 0, stream, q16, k16, v16, cu, h0, h0_index, num_h0,
                       o16, hT, r8, Hk, Hv, total);
  return hipGetLastError();
}

}  // namespace gdn
