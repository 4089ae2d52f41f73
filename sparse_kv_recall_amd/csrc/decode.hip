// Split-K decode attention over a paged bf16 KV cache: full, local (sinks + window)
// and block-list views, with the current token's commit fused in.
//
// What is computed (per request b, query head h, KV head g = h / (Hq/Hkv), key set S):
//   o_h = sum_{j in S} softmax_j(scale * <q_h, k_{g,j}>) v_{g,j}
// with S the Full view [0, n), the Local view [0, min(s,n)) u [max(.., n-w), n)
// (On-Demand Attention summary page, "Approach"; "Main results" for the window that
// counts the current token), the kept blocks of a Declarative-Attention keep-list
// (DA review page, section 3: block-granular mask by block-table rewrite), or the kept
// blocks of a declared DA mode, derived in the kernel from the declaration.
//
// How (gfx950):
//  * Work item = (request, KV head, split of consecutive tiles); a tile is one
//    16-position block of one KV head (4 KiB of K and 4 KiB of V). Every workgroup
//    derives the same plan from seq_lens / selectors, so no planning launch is needed.
//  * One workgroup = 8 waves sharing one work item; wave w takes tiles w, w+8, ... of the
//    split through a two-deep register ring (the next tile's loads in flight while the
//    current one is computed). K and V tiles are stored in the byte order of the MFMA
//    operands, so each lane issues plain coalesced 16-byte loads (1 KiB per wave
//    instruction) that are already its operand registers: no LDS staging, no shuffles.
//  * S = K q^T and O += V^T P^T run on the matrix cores. q (fp32) and p (fp32) are
//    split into bf16 hi + lo parts, so the products keep ~16 mantissa bits; the
//    accumulation is fp32. All query heads of a KV head share one read of K and V.
//  * Online softmax in base 2 (q pre-scaled by scale*log2 e), max reduced across the
//    four 16-lane rows with permlane swaps; waves combine through LDS; splits are merged by
//    the last workgroup to finish (atomic ticket per (request, KV head)) in registers,
//    in a fixed split order, so results are deterministic.
//  * Instances (decode_kernel<view, gated, single request, q/k finish, balanced order>):
//    one request runs straight-line code; the q/k-finish instances take a layer's raw
//    q/k/v projection and apply the per-head RMSNorm and rotary positions while staging
//    (Qwen3-family layer, for the weight-bearing decode step); the balanced-order
//    instances (the views launch, batches above 64) run ragged batches' work items
//    longest first, which changes which workgroup runs what, never the results.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "sk_internal.h"

namespace sk {
namespace {

enum { kFull = 0, kLocal = 1, kList = 2, kDecl = 3, kViews = 4 };
constexpr int kThreads = 64 * kWavesPerWG;
constexpr int kMinTilesPerSplit = 8;                   // small launches: many short splits
constexpr int kMaxSplits = 256;                     // splits per (request, KV head)
constexpr int kGridCap = 256;                       // decode workgroups per launch (one per CU)
constexpr int kBufferFlags = 0x00020000;  // raw buffer access, 32-bit data format (gfx9 word 3)
constexpr int kNonTemporal = 2;           // buffer load cache policy: non-temporal
constexpr int kTicketStride = 16;                   // words between ticket counters (small launches)
constexpr int kTabHeader = 3;                       // tile table row: length, sinks, window, then the tiles
constexpr int kMergeBatch = 48;                     // split accumulators loaded together in the merge
// Per-request views in one launch: work items fill at most this many rounds of the grid
// (4 x 256 workgroups = the items a workspace holds at the largest query group). Measured
// on the ragged batch of 32 (tokens/s against one launch per view): 2 rounds -2.5 %, 4
// rounds +1.8 %, 6 rounds +2.8 % (more items than the workspace holds at group 16), 8
// rounds +0.2 % (longer split merges).
constexpr int kViewRounds = 4;
// Largest batch that the workgroup-planned path runs in the balanced item order (ranking
// the requests' last splits takes about B^2 / 512 steps per thread).
constexpr int kOrderMaxBatch = 256;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x2 __attribute__((ext_vector_type(2)));

struct DecodeParams {
  const float* q;
  sk_paged_kv kv;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* sel;
  int sel_value;
  const int32_t* list_phys;
  const int32_t* list_cnt;
  const int32_t* list_num;
  float* out;
  int32_t* err;
  uint32_t* tickets;
  float* partials;
  int sinks;
  int window;
  float qscale;
  const int32_t* decl;  // declared view: {mode, focus_begin, focus_end, output_begin} per request
  int local_tokens;
  // Decoding from a layer's raw q/k/v projection (the kernel's QK instances): q holds
  // [B][Hq + 2 Hkv][128] fp32 rows (q heads, then k heads, then v heads); q and k heads
  // are RMS-normalised over their 128 values with gains g_q / g_k and rotated to position
  // n - 1 (pairs (i, i + 64), angle (n - 1) base^(-i/64)) before use; the current token's
  // k and v are rounded to bf16 for the commit.
  const uint16_t* g_q;
  const uint16_t* g_k;
  float qk_eps;
  float rope_base;
  // Local view from a step's tile table (oda_local_tiles): per request, the length, sinks
  // and window the table was built for, then the physical block of each Local tile;
  // tab_tiles = the largest Local tile count (its rows hold kTabHeader + tab_tiles words).
  // Null: no table.
  const int32_t* tab;
  int tab_tiles;
};

struct Tile {
  int phys, lo, hi;
};

template <bool HAS_SEL>
__device__ inline bool request_active(const DecodeParams& P, int b) {
  return !HAS_SEL || P.sel[b] == P.sel_value;
}

// Per-request views (MODE kViews): the selector value names the request's view, Full,
// Local or the gathered block list (SK_MODE_*); the view as one of kFull / kLocal /
// kList, or -1 for any other value (the request does not run).
__device__ inline int view_of(int sel) {
  return sel == SK_MODE_FULL ? int(kFull) : sel == SK_MODE_LOCAL ? int(kLocal) : sel == SK_MODE_BLOCKS ? int(kList) : -1;
}

// Kept blocks of a declared mode ([DA] sections 1 and 3) as at most two ascending,
// disjoint runs of logical blocks, [s0, s0 + l0) then [s1, s1 + l1), the same set (in the
// same order) as the keep mask of the declaration compacted into a list: global keeps every
// block below ceil(n/16); focus keeps [focus_begin, focus_end) and every block from
// output_begin on, both cut there; local keeps the blocks overlapping the last local_tokens
// positions; any other mode keeps nothing. n must be valid (1 .. max_blocks*16).
struct Runs {
  int s0, l0, s1, l1;
};
__device__ inline Runs declared_runs(const DecodeParams& P, int b, int n) {
  const int nb = (n + kBlock - 1) / kBlock;
  const int32_t* d = P.decl + 4 * int64_t(b);
  const int mode = d[0];
  int s0 = 0, e0 = 0, s1 = 0, e1 = 0;
  if (mode == SK_DA_GLOBAL) {
    e0 = nb;
  } else if (mode == SK_DA_LOCAL) {
    s0 = (n > P.local_tokens ? n - P.local_tokens : 0) / kBlock;
    e0 = nb;
  } else if (mode == SK_DA_FOCUS) {
    s0 = min(max(d[1], 0), nb);
    e0 = min(max(d[2], s0), nb);
    s1 = min(max(d[3], 0), nb);
    e1 = nb;
  }
  if (e0 <= s0) {  // first run empty: the second (possibly empty) one alone
    s0 = s1;
    e0 = e1;
    s1 = e1 = 0;
  }
  if (e1 <= s1) {
    s1 = e1 = 0;
  } else {
    if (s1 < s0) {  // ascending order
      const int ts = s0, te = e0;
      s0 = s1;
      e0 = e1;
      s1 = ts;
      e1 = te;
    }
    if (s1 <= e0) {  // overlapping or adjacent: one run
      e0 = max(e0, e1);
      s1 = e1 = 0;
    }
  }
  return Runs{s0, e0 - s0, s1, e1 - s1};
}

// listed: the request's entry of list_num (block-list view only); view: the request's view
// under MODE kViews (ignored otherwise)
template <int MODE>
__device__ inline int request_tiles(const DecodeParams& P, int b, int n, int listed, int view = MODE) {
  const int m = (MODE == kViews) ? view : MODE;
  if (m == kFull) return (n + kBlock - 1) / kBlock;
  if (m == kLocal) {
    int s_end = min(P.sinks, n);
    int a = max(s_end, n - P.window);
    int st = (s_end + kBlock - 1) / kBlock;
    int wt = (a < n) ? ((n - 1) / kBlock - a / kBlock + 1) : 0;
    return st + wt;
  }
  if (MODE == kDecl) {
    const Runs r = declared_runs(P, b, n);
    return r.l0 + r.l1;
  }
  (void)b;
  return min(max(listed, 0), P.kv.max_blocks);
}

// Local view tile i at length n: returns its logical block and sets [lo, hi), the valid
// positions in it (the sinks' blocks first, then the window's, cut at both ends).
__device__ inline int local_tile(const DecodeParams& P, int n, int i, int& lo, int& hi) {
  const int s_end = min(P.sinks, n);
  const int st = (s_end + kBlock - 1) / kBlock;
  if (i < st) {
    lo = 0;
    hi = min(kBlock, s_end - kBlock * i);
    return i;
  }
  const int a = max(s_end, n - P.window);
  const int j = i - st;
  const int lb = a / kBlock + j;
  lo = (j == 0) ? (a % kBlock) : 0;
  hi = min(kBlock, n - kBlock * lb);
  return lb;
}

template <int MODE>
__device__ inline Tile tile_at(const DecodeParams& P, int b, int n, int i, int view = MODE) {
  Tile t;
  const int32_t* bt = P.kv.block_tables + int64_t(b) * P.kv.max_blocks;
  const int m = (MODE == kViews) ? view : MODE;
  if (m == kFull) {
    t.lo = 0;
    t.hi = min(kBlock, n - kBlock * i);
    t.phys = bt[i];
  } else if (m == kLocal) {
    t.phys = bt[local_tile(P, n, i, t.lo, t.hi)];
  } else if (MODE == kDecl) {
    const Runs r = declared_runs(P, b, n);
    const int lb = (i < r.l0) ? r.s0 + i : r.s1 + (i - r.l0);
    t.lo = 0;
    t.hi = min(kBlock, n - kBlock * lb);
    t.phys = bt[lb];
  } else {
    int64_t o = int64_t(b) * P.kv.max_blocks + i;
    t.phys = P.list_phys[o];
    t.lo = 0;
    t.hi = min(max(P.list_cnt[o], 0), kBlock);
  }
  if (t.phys < 0 || t.phys >= P.kv.num_phys_blocks) {
    set_error(P.err, SK_DEVERR_BLOCK_ID);
    t.phys = 0;
    t.lo = t.hi = 0;
  }
  return t;
}

// The single-request plan for `tiles` tiles on `slots` split slots per KV head: tiles per
// split T (enough that the splits fit the slots after a reserve of one for rounding, at
// least kMinTilesPerSplit, at most kMaxSplits splits) and the splits; when those splits
// would leave more than a quarter of the slots idle, the smallest split size from
// tiles / slots up (its splits always fit the slots). The small-batch plan for one request.
__device__ inline void single_plan(int tiles, int slots, int& T, int& splits) {
  int budget = slots - (tiles > 0 ? 1 : 0);
  if (budget < 1) budget = 1;
  T = (tiles + budget - 1) / budget;
  const int T_cap = (tiles + kMaxSplits - 1) / kMaxSplits;
  if (T < T_cap) T = T_cap;
  if (T < kMinTilesPerSplit) T = kMinTilesPerSplit;
  splits = (tiles + T - 1) / T;
  if (4 * splits < 3 * slots) {
    int t = (tiles + slots - 1) / slots;
    if (t < T_cap) t = T_cap;
    if (t < kMinTilesPerSplit) t = kMinTilesPerSplit;
    if (t < T) {
      T = t;
      splits = (tiles + T - 1) / T;
    }
  }
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Split partials cross workgroups (and XCDs). They are written and read with
// device-scope relaxed atomic accesses, which gfx950 performs at the device coherence
// point (sc1), so publishing them needs only the completion of the stores before the
// ticket increment -- not an agent-scope fence, which would write back the whole L2.
__device__ inline void publish(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline float fetch_published(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wave reductions: DPP within each row of 16 lanes (swap neighbours, swap pairs, rotate
// by 4, rotate by 8), then the four row results read into scalar registers. The result
// is the same in every lane (taken from lanes 0, 16, 32, 48), so it is deterministic.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ inline float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp<kDppSwap1>(v));
  v = fmaxf(v, dpp<kDppSwap2>(v));
  v = fmaxf(v, dpp<kDppRor4>(v));
  v = fmaxf(v, dpp<kDppRor8>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ inline float wave_sum(float v) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppRor4>(v);
  v += dpp<kDppRor8>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Integer wave reductions and an inclusive prefix sum for the plan, all in registers
// (DPP). Scan: shift right by 1, 2, 4, 8 within each row of 16 (lanes shifted in from
// outside the row read 0), then add the last lane of row 0 to row 1 and of row 2 to
// row 3 (row broadcast 15), then lane 31 to rows 2 and 3 (row broadcast 31).
template <int CTRL, int ROWS = 0xF>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ inline int wave_sum_i(int v) {
  v += dpp_i<kDppSwap1>(v);
  v += dpp_i<kDppSwap2>(v);
  v += dpp_i<kDppRor4>(v);
  v += dpp_i<kDppRor8>(v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ inline int wave_max_i(int v) {
  v = max(v, dpp_i<kDppSwap1>(v));
  v = max(v, dpp_i<kDppSwap2>(v));
  v = max(v, dpp_i<kDppRor4>(v));
  v = max(v, dpp_i<kDppRor8>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
__device__ inline int wave_inclusive_scan(int v) {
  v += dpp_i<kDppShr1>(v);
  v += dpp_i<kDppShr2>(v);
  v += dpp_i<kDppShr4>(v);
  v += dpp_i<kDppShr8>(v);
  v += dpp_i<kDppBcast15, 0xA>(v);
  v += dpp_i<kDppBcast31, 0xC>(v);
  return v;
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) in
// registers, with gfx950's permlane swaps: the 16-lane swap trades the first operand's
// odd rows with the second operand's even rows, the 32-lane swap its upper half with
// the second operand's lower half; with the same value in both operands the two results
// hold a lane's value and its partner's. The copy goes through an empty asm statement so
// that the compiler sees two distinct operands: given one value twice it folds the
// swap's second result into the first, which the hardware does not do.
template <bool HALF>
__device__ inline void partner(float v, float& a, float& b) {
  unsigned x = __builtin_bit_cast(unsigned, v), y = x;
  asm volatile("" : "+v"(y));
  const auto r = HALF ? __builtin_amdgcn_permlane32_swap(x, y, false, false)
                      : __builtin_amdgcn_permlane16_swap(x, y, false, false);
  a = __builtin_bit_cast(float, unsigned(r[0]));
  b = __builtin_bit_cast(float, unsigned(r[1]));
}
__device__ inline float rows_max(float v) {
  float a, b;
  partner<false>(v, a, b);
  partner<true>(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ inline float rows_sum(float v) {
  float a, b;
  partner<false>(v, a, b);
  partner<true>(a + b, a, b);
  return a + b;
}

// One round of the split merge over nb <= NB consecutive splits, for one output element
// per lane (all lanes of the wave on one head): lane u loads the (m, l) of split u of the
// round (ml: the first split's m of this head; its l follows G floats later), every lane
// loads its element's accumulator of each split (acc: the first split's, splits `stride`
// floats apart), all in one round of independent loads. NB is the load count per lane:
// rounds are sized to the splits they hold, so that few splits issue few loads.
template <int NB>
__device__ inline void merge_round(const float* ml, const float* acc, uint32_t stride, int nb, int G, int lane,
                                   float& M, float& L, float& A) {
  const uint32_t mine = uint32_t(min(lane, nb - 1)) * stride;
  const float mv = fetch_published(ml + mine);
  const float lv = fetch_published(ml + mine + G);
  float as[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) as[u] = fetch_published(acc + uint32_t(min(u, nb - 1)) * stride);
  const float Mn = fmaxf(M, wave_max((lane < nb) ? mv : -INFINITY));
  const float Mu = (Mn == -INFINITY) ? 0.f : Mn;
  const float r = __builtin_amdgcn_exp2f(M - Mu);
  const float e = (lane < nb) ? __builtin_amdgcn_exp2f(mv - Mu) : 0.f;
  L = L * r + wave_sum(e * lv);
  A *= r;
  // weights past the round are zero and their (repeated) accumulators finite
#pragma unroll
  for (int u = 0; u < NB; ++u) A += lane_value(e, u) * as[u];
  M = Mn;
}

// s_waitcnt vmcnt(0): all of this wave's stores have completed (gfx9 counts stores in vmcnt).
__device__ inline void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ inline f32x4 mfma(u32x4 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), b, c, 0, 0, 0);
}

// 16x16x16 bf16: lane l supplies A[l%16][4(l/16)..+3] and B[4(l/16)..+3][l%16].
__device__ inline f32x4 mfma16(u32x2 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                  0, 0);
}

__device__ inline float bf16_to_f32(__bf16 x) { return float(x); }

// Writes token (n-1) of KV head g into the pool tile and returns nothing; used when
// the token's block is not attended (keep-list without it) or for invalid requests.
__device__ inline void commit_token_lanes(const DecodeParams& P, int b, int g, int n, int lane64) {
  const int Hkv = P.kv.num_kv_heads;
  int pos = n - 1;
  int phys = P.kv.block_tables[int64_t(b) * P.kv.max_blocks + pos / kBlock];
  if (phys < 0 || phys >= P.kv.num_phys_blocks) {
    set_error(P.err, SK_DEVERR_BLOCK_ID);
    return;
  }
  int t = pos % kBlock;
  size_t tile = (size_t(phys) * Hkv + g) * kTileBytes;
  uint8_t* kt = reinterpret_cast<uint8_t*>(P.kv.k_pool) + tile;
  uint8_t* vt = reinterpret_cast<uint8_t*>(P.kv.v_pool) + tile;
  const uint16_t* kn = P.k_new + (int64_t(b) * Hkv + g) * kHeadDim;
  const uint16_t* vn = P.v_new + (int64_t(b) * Hkv + g) * kHeadDim;
  if (lane64 < 16) {
    int d0 = lane64 * 8;
    *reinterpret_cast<u32x4*>(kt + (d0 >> 3) * 256 + t * 16) = *reinterpret_cast<const u32x4*>(kn + d0);
  }
  for (int d = lane64; d < kHeadDim; d += 64) {
    uint32_t off = (d >> 5) * 1024 + (t >> 2) * 256 + (d & 15) * 16 + ((d >> 4) & 1) * 8 + (t & 3) * 2;
    *reinterpret_cast<uint16_t*>(vt + off) = vn[d];
  }
}

// Replace position tl of a loaded tile (this lane's K / V operand registers) by the
// current token, staged in LDS as 64 words of K then 64 words of V (bf16 pairs).
__device__ inline void substitute_token(const uint32_t* s_new, int tl, int lane, u32x4 (&kr)[4], u32x4 (&vr)[4]) {
  const int m = lane & 15, grp = lane >> 4;
  if (m == tl) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int w = 4 * (4 * c + grp);  // dims 8*(4c+grp) .. +7
      kr[c] = u32x4{s_new[w], s_new[w + 1], s_new[w + 2], s_new[w + 3]};
    }
  }
  if (grp == (tl >> 2)) {
    const int j = tl & 3;
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(s_new + 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t val = vn[32 * c + 16 * h + m];
        uint32_t w = (j >> 1) ? (h ? vr[c].w : vr[c].y) : (h ? vr[c].z : vr[c].x);
        w = (j & 1) ? ((w & 0x0000FFFFu) | (val << 16)) : ((w & 0xFFFF0000u) | val);
        if (j >> 1) {
          if (h) vr[c].w = w; else vr[c].y = w;
        } else {
          if (h) vr[c].z = w; else vr[c].x = w;
        }
      }
    }
  }
}

// Store the current token (LDS copy) into position tl of the (phys, g) tiles.
__device__ inline void commit_from_lds(const DecodeParams& P, const uint32_t* s_new, int phys, int g, int tl,
                                       int lane) {
  const size_t tile = (size_t(phys) * P.kv.num_kv_heads + g) * kTileBytes;
  uint8_t* kt = reinterpret_cast<uint8_t*>(P.kv.k_pool) + tile;
  uint8_t* vt = reinterpret_cast<uint8_t*>(P.kv.v_pool) + tile;
  if (lane < 16)  // K: 16 chunks of 8 dims
    *reinterpret_cast<u32x4*>(kt + lane * 256 + tl * 16) =
        u32x4{s_new[4 * lane], s_new[4 * lane + 1], s_new[4 * lane + 2], s_new[4 * lane + 3]};
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(s_new + 64);
  for (int d = lane; d < kHeadDim; d += 64) {
    const uint32_t off = (d >> 5) * 1024 + (tl >> 2) * 256 + (d & 15) * 16 + ((d >> 4) & 1) * 8 + (tl & 3) * 2;
    *reinterpret_cast<uint16_t*>(vt + off) = vn[d];
  }
}

// QK instances: the layer's per-head q/k RMSNorm and rotary positions, applied while
// the q operands and the current token are staged. Every wave of the workgroup calls it
// (it holds a barrier). Wave 4, idle here otherwise, computes the 64 rotary (cos, sin)
// pairs of position n - 1 into LDS (angle in fp64, reduced to [-pi, pi] before its sine
// and cosine). Waves 0-3 hold the raw values of dims d0 .. d0 + 7 of q head qcol and
// publish them with their wave's share of the head's sum of squares; after the barrier
// each lane normalises its values and their rotary partners (dims d ^ 64, held by wave
// qc ^ 2), applies the gains and rotates. Waves 0 and 1 of the split that commits turn
// the raw k row (normalised within the wave, partner dims in lane ^ 32, rotated) and the
// raw v row into the bf16 words of s_new (word l: dims 2 l, 2 l + 1).
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ inline uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, __bf16(x)); }

__device__ inline void qk_finish_staged(const DecodeParams& P, int n, int wave, int lane, int qc, int qcol, int d0,
                                        int G, float (&xq)[8], const u32x4& gq, const u32x4& gqp, bool commits,
                                        f32x2 tok, uint32_t gk, float* scratch, uint32_t* s_new) {
  float* s_raw = scratch;                  // [G][128] raw q rows
  float* s_part = scratch + G * kHeadDim;  // [4][16] each wave's share of the heads' sums of squares
  float* s_rope = s_part + 64;             // [64] (cos, sin)
  if (wave == 4) {
    const double ang = double(n - 1) * exp2(-double(lane) / 64.0 * log2(double(P.rope_base)));
    const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    double sd, cd;
    sincos(red, &sd, &cd);
    s_rope[2 * lane] = float(cd);
    s_rope[2 * lane + 1] = float(sd);
  }
  if (wave < 4) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(xq[e], xq[e], ss);
    ss = rows_sum(ss);  // the wave's 32 dims of head qcol
    if (qcol < G) {
      *reinterpret_cast<f32x4*>(s_raw + qcol * kHeadDim + d0) = f32x4{xq[0], xq[1], xq[2], xq[3]};
      *reinterpret_cast<f32x4*>(s_raw + qcol * kHeadDim + d0 + 4) = f32x4{xq[4], xq[5], xq[6], xq[7]};
      if (lane < 16) s_part[qc * 16 + qcol] = ss;
    }
  }
  __syncthreads();
  if (wave < 4 && qcol < G) {
    const float tot = ((s_part[qcol] + s_part[16 + qcol]) + s_part[32 + qcol]) + s_part[48 + qcol];
    const float r = 1.f / sqrtf(tot / float(kHeadDim) + P.qk_eps);
    const f32x4 pa = *reinterpret_cast<const f32x4*>(s_raw + qcol * kHeadDim + (d0 ^ 64));
    const f32x4 pb = *reinterpret_cast<const f32x4*>(s_raw + qcol * kHeadDim + (d0 ^ 64) + 4);
    const float xp[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
    const uint32_t g8[4] = {gq.x, gq.y, gq.z, gq.w}, gp8[4] = {gqp.x, gqp.y, gqp.z, gqp.w};
    const int i0 = d0 & 63;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = s_rope[2 * (i0 + e)], sn = s_rope[2 * (i0 + e) + 1];
      const float v = xq[e] * r * ((e & 1) ? bf16_hi(g8[e >> 1]) : bf16_lo(g8[e >> 1]));
      const float vp = xp[e] * r * ((e & 1) ? bf16_hi(gp8[e >> 1]) : bf16_lo(gp8[e >> 1]));
      xq[e] = (d0 < 64) ? v * c - vp * sn : v * c + vp * sn;
    }
  }
  if (commits && wave < 2) {
    float o0 = tok.x, o1 = tok.y;
    if (wave == 0) {
      float ss = fmaf(tok.x, tok.x, tok.y * tok.y);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) ss += __shfl_xor(ss, o);  // same total in every lane
      const float r = 1.f / sqrtf(ss / float(kHeadDim) + P.qk_eps);
      const float v0 = tok.x * r * bf16_lo(gk), v1 = tok.y * r * bf16_hi(gk);
      float a, b;
      partner<true>(v0, a, b);
      const float p0 = (lane < 32) ? b : a;
      partner<true>(v1, a, b);
      const float p1 = (lane < 32) ? b : a;
      const int i0 = (2 * lane) & 63;
      const float c0 = s_rope[2 * i0], s0 = s_rope[2 * i0 + 1], c1 = s_rope[2 * i0 + 2], s1 = s_rope[2 * i0 + 3];
      o0 = (lane < 32) ? v0 * c0 - p0 * s0 : v0 * c0 + p0 * s0;
      o1 = (lane < 32) ? v1 * c1 - p1 * s1 : v1 * c1 + p1 * s1;
    }
    s_new[wave * 64 + lane] = bf16_bits(o0) | (bf16_bits(o1) << 16);
  }
}

// Zero the V halves of tokens outside [lo, hi) so that 0-weight tokens cannot bring in
// non-finite garbage (0 * NaN) through the PV product.
__device__ inline void mask_v(u32x4 (&vr)[4], int lo, int hi, int grp) {
  int t0 = 4 * grp;
  uint32_t m01 = ((t0 >= lo && t0 < hi) ? 0x0000FFFFu : 0u) | ((t0 + 1 >= lo && t0 + 1 < hi) ? 0xFFFF0000u : 0u);
  uint32_t m23 = ((t0 + 2 >= lo && t0 + 2 < hi) ? 0x0000FFFFu : 0u) | ((t0 + 3 >= lo && t0 + 3 < hi) ? 0xFFFF0000u : 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    vr[c].x &= m01;
    vr[c].y &= m23;
    vr[c].z &= m01;
    vr[c].w &= m23;
  }
}

// Loads the K and V tiles (4 KiB each) of one KV head of one physical block into this
// lane's MFMA operand registers: four 16-byte loads per tile, 1 KiB per wave instruction.
// The KV stream is read once per launch, so the loads carry the non-temporal hint.
// Branch-free: an empty descriptor (bad block id) points at block 0, whose positions the
// caller masks out, so the registers never have to be selected between two sources.
__device__ inline void load_tile(const uint8_t* kpool, const uint8_t* vpool, int phys, int g, int Hkv, int lane,
                                 u32x4 (&k)[4], u32x4 (&v)[4]) {
  const size_t off = (size_t(phys) * Hkv + g) * kTileBytes + 16 * lane;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    k[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kpool + off + 1024 * c));
    v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vpool + off + 1024 * c));
  }
}

// The tile at phys, or zeros without a memory access when ok is false: the loads go
// through buffer ranges that are empty then, so the number of loads in flight (which the
// waits count) does not depend on a branch.
__device__ inline void load_tile_if(const uint8_t* kpool, const uint8_t* vpool, int phys, int g, int Hkv, int lane,
                                    bool ok, u32x4 (&k)[4], u32x4 (&v)[4]) {
  const size_t base = (size_t(phys) * Hkv + g) * kTileBytes;
  const int bytes = __builtin_amdgcn_readfirstlane(ok ? int(kTileBytes) : 0);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kpool + base), 0, bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vpool + base), 0, bytes, kBufferFlags);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    k[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * lane + 1024 * c, 0, kNonTemporal));
    v[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, 16 * lane + 1024 * c, 0, kNonTemporal));
  }
}

// HAS_SEL: requests are filtered by sel[b] == sel_value (gated / per-request views).
// Without a selector a separate instance runs, so a profile tells gated launches
// (which exit at once on non-recall steps) apart from unconditional ones.
// SINGLE: a launch on one request. Its plan is the small-batch plan below for one request
// on the same grid (the same tiles per split, so the same work items and results as that
// request alone in a batch on the same grid), computed on the uniform length alone: no
// cross-lane reductions, scans or request search, which shortens the chain of
// instructions before the first tile is requested.
template <int MODE, bool HAS_SEL, bool SINGLE, bool QK = false, bool BAL = false, bool TAB = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams P) {
  constexpr int W = kWavesPerWG;
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = SINGLE ? 1 : P.kv.batch, Hkv = P.kv.num_kv_heads, Hq = P.kv.num_q_heads, G = Hq / Hkv;
  const int maxb = P.kv.max_blocks;
  const int acc_region = max(W * G * kHeadDim, 2 * kMaxSplits * G + 4 * kThreads);

  // LDS: q operands [4][2][64] x 16 B | current token K,V [128] words | acc [W][G][128] (merge scratch
  //      later) | m [W][16] | l [W][16] | tiles [B] | start [B+1] | len [B] | misc
  u32x4* s_q = reinterpret_cast<u32x4*>(smem);
  uint32_t* s_new = reinterpret_cast<uint32_t*>(smem + 4 * kThreads);  // current token: K [64] | V [64] words
  float* s_acc = smem + 4 * kThreads + 128;
  float* s_m = s_acc + acc_region;
  float* s_l = s_m + W * 16;
  int* s_tiles = reinterpret_cast<int*>(s_l + W * 16);
  int* s_start = s_tiles + B;
  int* s_len = s_start + B + 1;  // [B] sequence lengths (large batches)
  int* s_misc = s_len + B;  // [0] tile sum, [1] T, [2] active requests, [3] last flag, [4] max tiles
  int* s_view = s_misc + 8;  // [B] views of the requests (MODE kViews, large batches)
  // large batches in the balanced order: [B + 1] first position of each request's items
  // before its last splits, [B] its last split's tiles, [B] the request at each rank
  int* s_fstart = s_view + (MODE == kViews ? B : 0);
  int* s_rem = s_fstart + B + 1;
  int* s_byrank = s_rem + B;

  if (tid == 0) {
    s_misc[0] = 0;
    s_misc[2] = 0;
    s_misc[4] = 0;
  }
  // Gated launches: when no request is selected there is nothing to do (not even the
  // invalid-request handling, which only concerns selected requests), so every
  // workgroup leaves before touching the plan.
  // Small batches: lane b loads request b's length, selector and list length once, in one
  // round of loads (lanes past the batch read request 0 and ignore it).
  int l_len = 0, l_listed = 0, l_view = MODE;
  bool l_sel = true;
  // Local view from a tile table (TAB, single request): the row's header (the length, sinks
  // and window it was built for) and this wave's tile descriptors under the plan of the
  // largest Local tile count (the plan of every length from sinks + window on, unless the
  // window's alignment changes it), requested with the length, so that the first tiles can
  // be requested once it arrives. The item body takes them when the header and the plan
  // match, else it reads the block table as without a table. Every load here is
  // unconditional (an index past the wave's tiles is clamped into the row and its value not
  // used), so that all of them are requested before the first wait.
  int tab_phys = 0, tab_n = -1, tab_T = 0, tab_splits = 0, tab_s = -1, tab_w = -1;
  if (SINGLE) {  // uniform values, one round of loads
    const int n0 = P.kv.seq_lens[0];
    const int listed0 = (MODE == kList) ? P.list_num[0] : 0;
    const int sel0 = HAS_SEL ? P.sel[0] : 0;
    if constexpr (TAB) {
      tab_n = P.tab[0];
      tab_s = P.tab[1];
      tab_w = P.tab[2];
      single_plan(P.tab_tiles, int(gridDim.x) / Hkv, tab_T, tab_splits);
      const int ti = (int(blockIdx.x) % tab_splits) * tab_T + wave + lane * W;
      tab_phys = P.tab[kTabHeader + min(ti, P.tab_tiles - 1)];
    }
    l_len = __builtin_amdgcn_readfirstlane(n0);
    l_listed = __builtin_amdgcn_readfirstlane(listed0);
    if (HAS_SEL && __builtin_amdgcn_readfirstlane(sel0) != P.sel_value) return;
  } else if (B <= 64) {
    const int bl = (lane < B) ? lane : 0;
    l_len = P.kv.seq_lens[bl];
    if (MODE == kList || MODE == kViews) l_listed = P.list_num[bl];
    if (HAS_SEL) {
      if (MODE == kViews) {
        l_view = view_of(P.sel[bl]);
        l_sel = (lane < B) && l_view >= 0;
      } else {
        l_sel = (lane < B) && P.sel[bl] == P.sel_value;
      }
      if (__builtin_amdgcn_readfirstlane(__ballot(l_sel) != 0) == 0) return;
    }
  }

  // ---- plan: tiles per request, tiles per split, first work item of each request --
  // identical in every workgroup. Tiles per split: enough that the work items fit the
  // grid, never fewer than kMinTilesPerSplit, at most kMaxSplits splits per (request,
  // KV head).
  auto split_size = [&](int total, int active, int max_tiles) {
    int budget = int(gridDim.x) / Hkv - active;
    if (budget < 1) budget = 1;
    int T = (total + budget - 1) / budget;
    const int T_cap = (max_tiles + kMaxSplits - 1) / kMaxSplits;
    if (T < T_cap) T = T_cap;
    if (T < kMinTilesPerSplit) T = kMinTilesPerSplit;
    return T;
  };
  auto bad_request = [&](int b, int n, bool valid) {  // all-zero output row (+ commit if possible)
    set_error(P.err, valid ? SK_DEVERR_EMPTY : SK_DEVERR_SEQ_LEN);
    float* o = P.out + int64_t(b) * Hq * kHeadDim;
    for (int i = 0; i < Hq * kHeadDim; ++i) o[i] = 0.f;
    if (valid && P.k_new)
      for (int g = 0; g < Hkv; ++g)
        for (int l = 0; l < 64; ++l) commit_token_lanes(P, b, g, n, l);
  };
  int T, total_items;
  int w_tiles = 0, w_start = 0, w_len = 0;  // small batches: lane b holds request b's tiles,
                                             // first item and sequence length
  // Balanced item order (the loop at the end; instances with BAL, which the host picks for
  // the views launch and for batches above 64), used for the views and ragged batches:
  // small batches keep, in lane b, request b's items before its last splits (v_full, from
  // v_fstart in the execution order) and the rank of its last split's size; large batches
  // the same in LDS. n_full: the items before all last splits.
  bool balanced = false;
  int v_full = 0, v_fstart = 0, v_rank = 0, n_full = 0;
  if (SINGLE) {
    // the small-batch plan below for one request: the rounding reserve, then, when the
    // splits would leave more than a quarter of the slots idle, the smallest split size
    // from tiles / slots up (its splits always fit the slots)
    const int n = l_len;
    const bool valid = n >= 1 && n <= maxb * kBlock;
    const int tiles = valid ? request_tiles<MODE>(P, 0, n, l_listed) : 0;
    if (blockIdx.x == 0 && wave == 0 && lane == 0 && (!valid || tiles == 0)) bad_request(0, n, valid);
    int splits;
    single_plan(tiles, int(gridDim.x) / Hkv, T, splits);
    w_tiles = tiles;
    w_len = n;
    total_items = splits * Hkv;
  } else if (B <= 64) {
    // every wave plans on its own with register reductions; no workgroup barrier
    int tiles = 0;
    if (lane < B && l_sel) {
      const int n = l_len;
      const bool valid = n >= 1 && n <= maxb * kBlock;
      if (valid) tiles = request_tiles<MODE>(P, lane, n, l_listed, l_view);
      if (blockIdx.x == 0 && wave == 0 && (!valid || tiles == 0)) bad_request(lane, n, valid);
    }
    const int sum = wave_sum_i(tiles), act = wave_sum_i(tiles > 0), mx = wave_max_i(tiles);
    T = split_size(sum, act, mx);
    int splits = (tiles + T - 1) / T;  // this request's splits per KV head
    int x = wave_inclusive_scan(splits);
    // The budget above reserves one split per active request for rounding. With a few
    // long requests of similar length that reserve is mostly unused and can leave a
    // large part of the grid idle (16 requests of 2K tiles: half of it); with requests of
    // very different lengths the longest ones' splits set the launch time while the short
    // ones' single splits finish early. In both cases take the smallest tiles per split,
    // from total / slots up, whose splits fit the slots. (Not for one request or equal
    // lengths that already fill most of the grid: equal splits that start at aligned
    // offsets and move in lockstep measured slower there.)
    const int slots = int(gridDim.x) / Hkv;
    const int used = __builtin_amdgcn_readlane(x, 63);
    if (4 * used < 3 * slots || (used < slots && mx * act > 2 * sum)) {
      auto count = [&](int t) { return wave_sum_i((tiles + t - 1) / t); };
      int t = (sum + slots - 1) / slots;
      const int t_cap = (mx + kMaxSplits - 1) / kMaxSplits;
      if (t < t_cap) t = t_cap;
      if (t < kMinTilesPerSplit) t = kMinTilesPerSplit;
      for (int k = 0; k < 8 && t < T && count(t) > slots; ++k) t += (t >> 3) + 1;
      if (t < T && count(t) <= slots) {
        T = t;
        splits = (tiles + T - 1) / T;
        x = wave_inclusive_scan(splits);
      }
    }
    if (MODE == kViews && mx * act > 2 * sum) {
      // Views of different sizes in one launch: the reserve above gives every running
      // request a slot, so with as many requests as slots each gets one split and the
      // longest Full views set the launch time. Size the splits instead so that the work
      // items fill at most kViewRounds rounds of the grid: a workgroup then takes about
      // that many items of at most T tiles, close to an even share.
      auto count = [&](int t) { return wave_sum_i((tiles + t - 1) / t); };
      const int cap = kViewRounds * slots;
      int t = (sum + cap - 1) / cap;
      const int t_cap = (mx + kMaxSplits - 1) / kMaxSplits;
      if (t < t_cap) t = t_cap;
      if (t < kMinTilesPerSplit) t = kMinTilesPerSplit;
      for (int k = 0; k < 16 && t < T && count(t) > cap; ++k) t += (t >> 3) + 1;
      if (t < T && count(t) <= cap) {  // within the items the workspace holds
        T = t;
        splits = (tiles + T - 1) / T;
        x = wave_inclusive_scan(splits);
      }
    }
    w_tiles = tiles;
    w_len = (lane < B) ? l_len : 0;
    w_start = (x - splits) * Hkv;
    total_items = __builtin_amdgcn_readlane(x, 63) * Hkv;
    balanced = BAL && (MODE == kViews || mx * act > 2 * sum);
    if (BAL && balanced) {
      // Execution order of the items (the loop at the end): every request's splits but
      // its last first, then the last splits, largest first (ties by request), so that
      // the short items fill in at the end instead of lengthening some workgroups' share.
      v_full = (splits > 0) ? (splits - 1) * Hkv : 0;
      const int f = wave_inclusive_scan(v_full);
      v_fstart = f - v_full;
      n_full = __builtin_amdgcn_readlane(f, 63);
      const int rem = (splits > 0) ? tiles - (splits - 1) * T : -1;
      int rank = 0;
      for (int o = 0; o < 64; ++o) {
        const int ro = __builtin_amdgcn_readlane(rem, o);
        rank += (ro > rem || (ro == rem && o < lane)) ? 1 : 0;
      }
      v_rank = rank;
    }
  } else {
    __syncthreads();
    int my_sum = 0, my_active = 0, my_max = 0;
    for (int b = tid; b < B; b += blockDim.x) {
      int tiles = 0;
      const int view = (MODE == kViews) ? view_of(P.sel[b]) : MODE;
      if (MODE == kViews) s_view[b] = view;
      if (MODE == kViews ? view >= 0 : request_active<HAS_SEL>(P, b)) {
        const int n = P.kv.seq_lens[b];
        const bool valid = n >= 1 && n <= maxb * kBlock;
        if (valid) tiles = request_tiles<MODE>(P, b, n, (MODE == kList || MODE == kViews) ? P.list_num[b] : 0, view);
        if (blockIdx.x == 0 && (!valid || tiles == 0)) bad_request(b, n, valid);
      }
      s_tiles[b] = tiles;
      s_len[b] = P.kv.seq_lens[b];
      my_sum += tiles;
      my_active += tiles > 0;
      my_max = max(my_max, tiles);
    }
    if (my_sum) atomicAdd(&s_misc[0], my_sum);
    if (my_active) atomicAdd(&s_misc[2], my_active);
    if (my_max) atomicMax(&s_misc[4], my_max);
    __syncthreads();
    if (tid == 0) {
      int t = split_size(s_misc[0], s_misc[2], s_misc[4]);
      if (BAL && B <= kOrderMaxBatch && s_misc[4] * s_misc[2] > 2 * s_misc[0]) {
        // ragged lengths in the balanced order: split the long requests too, within the
        // items a workspace holds (kTargetItems beyond one item per request and KV head)
        const int per_head = max(1, kTargetItems / Hkv);
        int t2 = (s_misc[0] + per_head - 1) / per_head;
        const int t_cap = (s_misc[4] + kMaxSplits - 1) / kMaxSplits;
        if (t2 < t_cap) t2 = t_cap;
        if (t2 < kMinTilesPerSplit) t2 = kMinTilesPerSplit;
        if (t2 < t) t = t2;
      }
      s_misc[1] = t;
    }
    __syncthreads();
    T = s_misc[1];
    if (wave == 0) {
      int carry = 0;
      for (int base = 0; base < B; base += 64) {
        const int b = base + lane;
        const int items = (b < B) ? ((s_tiles[b] + T - 1) / T) * Hkv : 0;
        const int x = wave_inclusive_scan(items);
        if (b < B) s_start[b] = carry + x - items;
        carry += __builtin_amdgcn_readlane(x, 63);
      }
      if (lane == 0) s_start[B] = carry;
    }
    __syncthreads();
    total_items = s_start[B];
    balanced = BAL && B <= kOrderMaxBatch && (MODE == kViews || s_misc[4] * s_misc[2] > 2 * s_misc[0]);
    if (BAL && balanced) {  // the same order as for small batches, ranked in LDS
      if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < B; base += 64) {
          const int b = base + lane;
          const int sp = (b < B) ? (s_tiles[b] + T - 1) / T : 0;
          const int full = (sp > 0) ? (sp - 1) * Hkv : 0;
          const int x = wave_inclusive_scan(full);
          if (b < B) {
            s_fstart[b] = carry + x - full;
            s_rem[b] = (sp > 0) ? s_tiles[b] - (sp - 1) * T : -1;
          }
          carry += __builtin_amdgcn_readlane(x, 63);
        }
        if (lane == 0) s_fstart[B] = carry;
      }
      __syncthreads();
      for (int b = tid; b < B; b += blockDim.x) {
        const int rem = s_rem[b];
        if (rem < 0) continue;
        int rank = 0;
        for (int o = 0; o < B; ++o) {
          const int ro = s_rem[o];
          rank += (ro > rem || (ro == rem && o < b)) ? 1 : 0;
        }
        s_byrank[rank] = b;
      }
      __syncthreads();
      n_full = s_fstart[B];
    }
  }

  // Items in workgroup order. The dispatcher deals workgroups round-robin over the 8
  // XCDs, so a launch with fewer items than workgroups still spreads over all of them;
  // partials and tickets go through device-coherent stores and loads, so the XCD that
  // merges a (request, KV head) does not need to be the one that wrote its partials.
  const int item_first = int(blockIdx.x);

  // Ticket counters kTicketStride words apart (a 64-byte line each) when the launch's
  // (request, KV head) pairs fit the ticket region that way: the ticket atomics of all
  // splits arrive together at the end of a launch, and counters sharing a line are updated
  // one after another (measured: Local view 9.43 -> 9.20 us, 12.5 % block list 17.6 ->
  // 16.8 us per launch).
  const int ticket_stride = (int64_t(B) * Hkv * kTicketStride <= kMaxTickets) ? kTicketStride : 1;
  const int ncol = lane & 15, grp = lane >> 4;
  const uint8_t* kpool = reinterpret_cast<const uint8_t*>(P.kv.k_pool);
  const uint8_t* vpool = reinterpret_cast<const uint8_t*>(P.kv.v_pool);

  // One work item. A single-request launch has at most one item per workgroup (its plan
  // never makes more items than the grid has workgroups; the host picks that instance only
  // for grids of at least two workgroups per KV head), so it runs the body once, as
  // straight-line code: kept in a loop, the compiler hoists the loop-invariant values and
  // spills them to vector lanes at the loop head, about 500 instructions before the first
  // request of a launch.
  auto item_body = [&](const int item) {
    // locate the request: the one whose item range holds `item` (it has items)
    int b, tiles_b, item_base, n, view = MODE;  // view: the request's view under kViews
    if (SINGLE) {
      b = 0;
      tiles_b = w_tiles;
      n = w_len;
      item_base = 0;
    } else if (B <= 64) {
      const int end = w_start + ((w_tiles + T - 1) / T) * Hkv;
      b = __builtin_amdgcn_readfirstlane(__popcll(__ballot(lane < B && end <= item)));
      tiles_b = __builtin_amdgcn_readlane(w_tiles, b);
      n = __builtin_amdgcn_readlane(w_len, b);
      item_base = __builtin_amdgcn_readlane(w_start, b);
      if (MODE == kViews) view = __builtin_amdgcn_readlane(l_view, b);
    } else {
      int lo_b = 0, hi_b = B - 1;
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (s_start[mid] <= item) lo_b = mid; else hi_b = mid - 1;
      }
      b = lo_b;
      tiles_b = s_tiles[b];
      n = s_len[b];
      item_base = s_start[b];
      if (MODE == kViews) view = s_view[b];
    }
    const int splits = (tiles_b + T - 1) / T;
    const int local = item - item_base;
    const int g = local / splits, split = local % splits;
    const int t_begin = split * T, t_end = min(t_begin + T, tiles_b);

    // Tiles of this wave: wave, wave + W, ... of the split. Their descriptors (physical
    // block, valid range; lane r for tile r of a chunk of 64) are requested first: the
    // first tile's request waits for them, and the loads issued after them (q rows, the
    // commit lookups, the current token) stay in flight meanwhile. The descriptors are
    // bounded by the wave's tiles, the commit tile included (a descriptor loaded and not
    // used costs nothing).
    const int my_tiles = (t_end - t_begin > wave) ? (t_end - t_begin - wave + W - 1) / W : 0;
    int dphys = 0, dlohi = 0;
    auto load_desc = [&](int c0) {
      const int ti = t_begin + wave + (c0 + lane) * W;
      Tile tt = Tile{0, 0, 0};
      if (c0 + lane < my_tiles) tt = tile_at<MODE>(P, b, n, ti, view);
      dphys = tt.phys;
      dlohi = tt.lo | (tt.hi << 8);
    };
    // List views: the current token's block and the list's last entry, requested with the
    // descriptors (whose wait then covers them) rather than after them.
    int lk_token = 0, lk_last = 0;
    if ((MODE == kList || MODE == kViews) && (QK || P.k_new)) {
      if (MODE == kList || view == kList) {
        lk_token = P.kv.block_tables[int64_t(b) * maxb + (n - 1) / kBlock];
        lk_last = P.list_phys[int64_t(b) * maxb + tiles_b - 1];
      }
    }
    bool from_tab = false;
    if constexpr (TAB)  // the table was built for this length, sinks and window, and this plan
      from_tab = (tab_n == n) & (tab_s == P.sinks) & (tab_w == P.window) & (T == tab_T) & (splits == tab_splits);
    if (from_tab) {  // the table's blocks, checked as tile_at checks the block table's
      int lo = 0, hi = 0, phys = 0;
      if (lane < my_tiles) {
        phys = tab_phys;
        local_tile(P, n, t_begin + wave + lane * W, lo, hi);
        if (phys < 0 || phys >= P.kv.num_phys_blocks) {
          set_error(P.err, SK_DEVERR_BLOCK_ID);
          phys = 0;
          lo = hi = 0;
        }
      }
      dphys = phys;
      dlohi = lo | (hi << 8);
    } else {
      load_desc(0);
    }

    // q rows of the G heads of KV head g for the operand staging below. Waves 0-3 load
    // them (wave c the dims of chunk c) and stage both bf16 parts; waves 4-7 request
    // nothing here, so the workgroup's first round of loads stays small. Lanes past the G
    // heads read head 0 (and stage zeros).
    const int qc = wave & 3, qcol = lane & 15, qgrp = lane >> 4;
    const int q_rows = QK ? Hq + 2 * Hkv : Hq;  // rows of one request in P.q
    const int d0 = 8 * (4 * qc + qgrp);         // this lane's first q dim
    const float* qrow = P.q + (int64_t(b) * q_rows + g * G + (qcol < G ? qcol : 0)) * kHeadDim + d0;
    f32x4 qa0 = {0.f, 0.f, 0.f, 0.f}, qa1 = {0.f, 0.f, 0.f, 0.f};
    u32x4 gq = {0u, 0u, 0u, 0u}, gqp = {0u, 0u, 0u, 0u};  // QK: gains of dims d0.. and of their partners
    if (wave < 4) {
      qa0 = *reinterpret_cast<const f32x4*>(qrow);
      qa1 = *reinterpret_cast<const f32x4*>(qrow + 4);
      if (QK) {
        gq = *reinterpret_cast<const u32x4*>(P.g_q + d0);
        gqp = *reinterpret_cast<const u32x4*>(P.g_q + (d0 ^ 64));
      }
    }

    // which tile receives the current token (-1: none attended here)
    int commit_tile = -1;
    const int tl = (n - 1) % kBlock;
    if (QK || P.k_new) {
      const int m = (MODE == kViews) ? view : MODE;
      if (m == kFull || m == kLocal) {
        commit_tile = tiles_b - 1;
      } else if (MODE == kDecl) {
        // the current token's block is attended when it is the last kept block
        const Runs r = declared_runs(P, b, n);
        const int last_blk = (r.l1 > 0) ? r.s1 + r.l1 - 1 : r.s0 + r.l0 - 1;
        if (last_blk == (n - 1) / kBlock) commit_tile = tiles_b - 1;
        else if (split == 0 && wave == 0) commit_token_lanes(P, b, g, n, lane);
      } else {
        if (lk_last == lk_token) commit_tile = tiles_b - 1;
        else if (split == 0 && wave == 0) commit_token_lanes(P, b, g, n, lane);
      }
    }

    // The tile that receives the current token (the request's last tile) is the owning
    // wave's last tile; its key and value come from LDS, staged below together with q, so
    // the pipeline never waits on them.
    const bool split_commits = commit_tile >= t_begin && commit_tile < t_end;
    const bool own_commit = split_commits && (commit_tile - t_begin) % W == wave;
    const int loop_tiles = my_tiles - (own_commit ? 1 : 0);
    // the current token's K (wave 0) and V (wave 1) words, staged in LDS below when this
    // split receives the token; the uniform branch sits before a full wait (the descriptor
    // loads below are waited for before the first tile is requested), so it costs no
    // wait-count precision
    uint32_t tok_word = 0u;
    f32x2 tok_raw = {0.f, 0.f};  // QK: dims 2 lane, 2 lane + 1 of the projection's k (wave 0) or v (wave 1) row
    uint32_t gk = 0u;            // QK: their k gains
    if (split_commits && wave < 2) {
      if (QK) {
        const float* row = P.q + (int64_t(b) * q_rows + Hq + wave * Hkv + g) * kHeadDim;
        tok_raw = reinterpret_cast<const f32x2*>(row)[lane];
        if (wave == 0) gk = reinterpret_cast<const uint32_t*>(P.g_k)[lane];
      } else {
        tok_word =
            reinterpret_cast<const uint32_t*>((wave ? P.v_new : P.k_new) + (int64_t(b) * Hkv + g) * kHeadDim)[lane];
      }
    }

    // q -> MFMA B operands (hi and lo bf16 parts), staged in LDS: entry (c, part, lane) holds
    // dims 8*(4c + lane/16) .. +7 of head lane%16. The wave's first tile is requested
    // before the q rows are used, so its latency overlaps the staging. A wave without tiles
    // requests block 0 of the pool and never uses it, so the request needs no branch.
    u32x4 k0[4], v0[4], k1[4], v1[4];
    load_tile(kpool, vpool, __builtin_amdgcn_readfirstlane(dphys), g, Hkv, lane, k0, v0);
    if (QK) {
      float xq[8] = {qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
      qk_finish_staged(P, n, wave, lane, qc, qcol, d0, G, xq, gq, gqp, split_commits, tok_raw, gk, s_acc, s_new);
      qa0 = f32x4{xq[0], xq[1], xq[2], xq[3]};
      qa1 = f32x4{xq[4], xq[5], xq[6], xq[7]};
    } else if (split_commits && tid < 128) {
      s_new[tid] = tok_word;
    }
    if (wave < 4) {
      const float x[8] = {qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
      bf16x8 oh, ol;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = x[i] * P.qscale;
        const __bf16 hi = __bf16(v);
        oh[i] = hi;
        ol[i] = __bf16(v - bf16_to_f32(hi));
      }
      const u32x4 z = {0u, 0u, 0u, 0u};
      s_q[qc * 128 + lane] = (qcol < G) ? __builtin_bit_cast(u32x4, oh) : z;
      s_q[qc * 128 + 64 + lane] = (qcol < G) ? __builtin_bit_cast(u32x4, ol) : z;
    }
    if constexpr (MODE == kLocal) {
      // the wave's second tile too, before the barrier (its waves hold one or two tiles)
      load_tile_if(kpool, vpool, __builtin_amdgcn_readlane(dphys, 1), g, Hkv, lane, loop_tiles >= 2, k1, v1);
    }
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto process = [&](u32x4 (&k)[4], u32x4 (&v)[4], int lohi) {
      const int lo = lohi & 255, hi = lohi >> 8;
      mask_v(v, lo, hi, grp);
      // S = K q^T: lane holds positions 4*grp + jj of head ncol
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) s = mfma(k[c], __builtin_bit_cast(bf16x8, s_q[c * 128 + lane]), s);
#pragma unroll
      for (int c = 0; c < 4; ++c) s = mfma(k[c], __builtin_bit_cast(bf16x8, s_q[c * 128 + 64 + lane]), s);
      float sv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = 4 * grp + jj;
        sv[jj] = (t >= lo && t < hi) ? s[jj] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = rows_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float pv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pv[jj] = __builtin_amdgcn_exp2f(sv[jj] - m_use);
      l_run = l_run * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
      m_run = m_new;
      bf16x4 ph, pl;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        __bf16 h16 = __bf16(pv[jj]);
        ph[jj] = h16;
        pl[jj] = __bf16(pv[jj] - bf16_to_f32(h16));
      }
      // O^T += V^T P^T, 16 dims at a time: the lane's V operand is 4 positions of one dim
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        const int c = dc >> 1;
        const u32x2 a = (dc & 1) ? u32x2{v[c].z, v[c].w} : u32x2{v[c].x, v[c].y};
        acc[dc] *= alpha;
        acc[dc] = mfma16(a, ph, acc[dc]);
        acc[dc] = mfma16(a, pl, acc[dc]);
      }
    };

    // Pipelined loop over chunks of up to 64 tiles: lane r holds the descriptor (physical
    // block, valid range) of chunk tile r; two tile buffers alternate, so the next tile is
    // in flight while this one is computed (a deeper ring measured slower: more loads in
    // flight per wave only added queueing). The loop body has no data-dependent branch: a
    // fetch that is conditional inside it makes the compiler wait for every load in flight
    // before the next tile, which cost the 128K Full view 3 %. The last pair of an even
    // chunk is therefore peeled, so that no fetch follows it. (Clamping that fetch to the
    // chunk's last tile instead re-requests a tile whose first request is still in flight,
    // and both go to HBM: 15 % more traffic for splits of 34 tiles, i.e. 4 or 5 per wave.)
    // The Local view's waves hold one or two tiles at batch 1: it requests a wave's second
    // tile before the staging barrier, together with the first (the wave holding two
    // tiles was the last to finish: its second request waited for the barrier), and
    // fetches past the chunk's end through empty buffer ranges instead of peeling the
    // last pair (whose larger code cost it 0.13 us per launch).
    for (int c0 = 0; c0 < loop_tiles; c0 += 64) {
      const int nt = min(64, loop_tiles - c0);
      const int last = nt - 1;
#define SK_FETCH(K, V, J) load_tile(kpool, vpool, __builtin_amdgcn_readlane(dphys, min((J), last)), g, Hkv, lane, K, V)
#define SK_LOHI(J) __builtin_amdgcn_readlane(dlohi, (J))
      if (c0 > 0) {
        load_desc(c0);
        SK_FETCH(k0, v0, 0);
      }
      int j = 0;
      if constexpr (MODE == kLocal) {
#define SK_FETCH_IF(K, V, J) \
  load_tile_if(kpool, vpool, __builtin_amdgcn_readlane(dphys, min((J), last)), g, Hkv, lane, (J) <= last, K, V)
        if (c0 > 0) SK_FETCH_IF(k1, v1, 1);  // the first chunk's was requested before the staging barrier
        for (; j + 2 <= nt; j += 2) {
          process(k0, v0, SK_LOHI(j));
          SK_FETCH_IF(k0, v0, j + 2);
          process(k1, v1, SK_LOHI(j + 1));
          SK_FETCH_IF(k1, v1, j + 3);
        }
        if (j < nt) process(k0, v0, SK_LOHI(j));
#undef SK_FETCH_IF
      } else {
        for (; j + 2 < nt; j += 2) {
          SK_FETCH(k1, v1, j + 1);
          process(k0, v0, SK_LOHI(j));
          SK_FETCH(k0, v0, j + 2);
          process(k1, v1, SK_LOHI(j + 1));
        }
        if (j + 2 == nt) {
          SK_FETCH(k1, v1, j + 1);
          process(k0, v0, SK_LOHI(j));
          process(k1, v1, SK_LOHI(j + 1));
        } else if (j < nt) {
          process(k0, v0, SK_LOHI(j));
        }
      }
#undef SK_FETCH
#undef SK_LOHI
    }
    if (own_commit) {
      // the request's last tile: attend with the current token substituted from LDS, then
      // write the token into its slot of the pool. When it is the wave's only tile, the
      // first request above already fetched it (lane 0's descriptor is that tile).
      Tile tt;
      if (loop_tiles == 0) {
        const int lohi = __builtin_amdgcn_readfirstlane(dlohi);
        tt = Tile{__builtin_amdgcn_readfirstlane(dphys), lohi & 255, lohi >> 8};
      } else {
        tt = tile_at<MODE>(P, b, n, commit_tile, view);
        load_tile(kpool, vpool, tt.phys, g, Hkv, lane, k0, v0);
      }
      substitute_token(s_new, tl, lane, k0, v0);
      process(k0, v0, tt.lo | (tt.hi << 8));
      if (tt.hi > tt.lo) commit_from_lds(P, s_new, tt.phys, g, tl, lane);
    }

    // ---- combine the waves of this workgroup
    l_run = rows_sum(l_run);
    if (ncol < G) {
#pragma unroll
      for (int dc = 0; dc < 8; ++dc)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s_acc[(wave * G + ncol) * kHeadDim + 16 * dc + 4 * grp + jj] = acc[dc][jj];
      if (grp == 0) {
        s_m[wave * 16 + ncol] = m_run;
        s_l[wave * 16 + ncol] = l_run;
      }
    }
    __syncthreads();
    float* part = P.partials + size_t(item) * G * (kHeadDim + 2);
    for (int idx = tid; idx < G * kHeadDim; idx += blockDim.x) {
      const int h = idx >> 7, d = idx & (kHeadDim - 1);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w * 16 + h]);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        float e = __builtin_amdgcn_exp2f(s_m[w * 16 + h] - Mu);
        L += s_l[w * 16 + h] * e;
        A += s_acc[(w * G + h) * kHeadDim + d] * e;
      }
      if (splits == 1) {
        P.out[(int64_t(b) * Hq + g * G + h) * kHeadDim + d] = (L > 0.f) ? A / L : 0.f;
      } else {
        publish(part + h * kHeadDim + d, A);
        if (d == 0) {
          publish(part + G * kHeadDim + h, M);
          publish(part + G * (kHeadDim + 1) + h, L);
        }
      }
    }

    // ---- the last split of (b, g) to finish merges all splits, in split order
    if (splits > 1) {
      // The partials were written with device-coherent stores; every wave waits for its
      // stores to complete before the barrier, then one thread takes the ticket. The last
      // arrival reads the partials with device-coherent loads. No L2 write-back is needed.
      wait_stores();
      __syncthreads();
      if (tid == 0) {
        unsigned prev = atomicAdd(&P.tickets[(b * Hkv + g) * ticket_stride], 1u);
        s_misc[3] = (prev == unsigned(splits - 1));
      }
      __syncthreads();
      if (s_misc[3]) {
        // Merge in split order, kMergeBatch splits at a time, without LDS: all 64 lanes of
        // a wave work on one head, lane u holds the (m, l) of split u of the batch, and
        // each lane loads the accumulators of its output element for the whole batch in
        // the same round of independent loads. The batch maximum and weighted sum of l
        // are wave reductions; lane u's weight is broadcast (readlane) to scale split u's
        // accumulator, in split order.
        const int S = splits;
        const uint32_t stride = uint32_t(G) * (kHeadDim + 2);  // floats per split partial
        const float* base = P.partials + size_t(item_base + g * splits) * stride;
        for (int idx = tid; idx < G * kHeadDim; idx += blockDim.x) {
          const int h = idx >> 7;  // uniform in the wave
          float M = -INFINITY, L = 0.f, A = 0.f;
          for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
            const int nb = min(kMergeBatch, S - s0);
            const uint32_t ml = uint32_t(s0) * stride + G * kHeadDim + h;
            const float* acc0 = base + (uint32_t(s0) * stride + uint32_t(idx));
            if (nb <= 16)
              merge_round<16>(base + ml, acc0, stride, nb, G, lane, M, L, A);
            else if (nb <= 32)
              merge_round<32>(base + ml, acc0, stride, nb, G, lane, M, L, A);
            else
              merge_round<kMergeBatch>(base + ml, acc0, stride, nb, G, lane, M, L, A);
          }
          P.out[(int64_t(b) * Hq + g * G + h) * kHeadDim + (idx & (kHeadDim - 1))] = (L > 0.f) ? A / L : 0.f;
        }
        if (tid == 0) P.tickets[(b * Hkv + g) * ticket_stride] = 0u;
      }
    }
    __syncthreads();
  };
  if constexpr (SINGLE) {
    if (item_first < total_items) item_body(item_first);
  } else if constexpr (!BAL) {
    for (int item = item_first; item < total_items; item += gridDim.x) item_body(item);
  } else {
    // Position i of the execution order -> the item (its partials keep the item's slot,
    // and merges run in split order, so results do not depend on the order). Rounds of the
    // grid alternate direction, so a workgroup that takes a larger item in one round
    // takes a smaller one in the next.
    auto item_at = [&](const int i) {
      int b, sp;
      if (B <= 64) {  // per-request values in lane b
        if (i < n_full) {
          b = __builtin_amdgcn_readfirstlane(__popcll(__ballot(lane < B && v_fstart + v_full <= i)));
          sp = (__builtin_amdgcn_readlane(w_tiles, b) + T - 1) / T;
          const int local = i - __builtin_amdgcn_readlane(v_fstart, b);
          return __builtin_amdgcn_readlane(w_start, b) + (local / (sp - 1)) * sp + local % (sp - 1);
        }
        b = __builtin_amdgcn_readfirstlane(int(__builtin_ctzll(__ballot(lane < B && v_rank == (i - n_full) / Hkv))));
        sp = (__builtin_amdgcn_readlane(w_tiles, b) + T - 1) / T;
        return __builtin_amdgcn_readlane(w_start, b) + ((i - n_full) % Hkv) * sp + sp - 1;
      }
      if (i < n_full) {  // the request whose items before its last splits hold position i
        int lo_b = 0, hi_b = B - 1;
        while (lo_b < hi_b) {
          const int mid = (lo_b + hi_b + 1) >> 1;
          if (s_fstart[mid] <= i) lo_b = mid; else hi_b = mid - 1;
        }
        sp = (s_tiles[lo_b] + T - 1) / T;
        const int local = i - s_fstart[lo_b];
        return s_start[lo_b] + (local / (sp - 1)) * sp + local % (sp - 1);
      }
      b = s_byrank[(i - n_full) / Hkv];
      sp = (s_tiles[b] + T - 1) / T;
      return s_start[b] + ((i - n_full) % Hkv) * sp + sp - 1;
    };
    // one loop for both orders, so that the item body is compiled once
    const int grid = int(gridDim.x);
    for (int r = 0; r * grid < total_items; ++r) {
      const int i = r * grid + ((balanced && (r & 1)) ? grid - 1 - item_first : item_first);
      if (i < total_items) item_body(balanced ? item_at(i) : i);
    }
  }
}

// Keep-mask -> ascending list of (physical block, valid positions). One thread per
// logical block, 256 blocks per workgroup, many workgroups per request: a workgroup
// counts the kept blocks of all mask words before its range (one wave, popcounts),
// ranks its own blocks with ballots, and writes its entries coalesced. The workgroup
// that holds block ceil(n/16)-1 writes the count.
__global__ __launch_bounds__(256) void gather_kernel(sk_paged_kv kv, const uint32_t* __restrict__ mask,
                                                     const int32_t* __restrict__ sel, int sel_value,
                                                     int32_t* __restrict__ gathered, int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ num_kept, int32_t* err) {
  __shared__ int s_wave[4];
  __shared__ int s_prefix;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (sel && sel[b] != sel_value) return;
  const int n = kv.seq_lens[b];
  const int maxb = kv.max_blocks;
  if (n < 1 || n > maxb * kBlock) {
    if (blockIdx.x == 0 && tid == 0) {
      num_kept[b] = 0;
      set_error(err, SK_DEVERR_SEQ_LEN);
    }
    return;
  }
  const int nb = (n + kBlock - 1) / kBlock;
  const int base = blockIdx.x * 256;
  if (base >= nb) return;
  const uint32_t* mrow = mask + int64_t(b) * ((maxb + 31) / 32);
  if (wave == 0) {  // kept blocks before this workgroup's range (all full words)
    int c = 0;
    for (int w = lane; w < base / 32; w += 64) c += __popc(mrow[w]);
    c = wave_sum_i(c);
    if (lane == 0) s_prefix = c;
  }
  const int blk = base + tid;
  const bool kept = blk < nb && ((mrow[blk >> 5] >> (blk & 31)) & 1u);
  const uint64_t bal = __ballot(kept);
  const int rank = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(bal);
  __syncthreads();
  int pos = s_prefix + rank;
  for (int i = 0; i < wave; ++i) pos += s_wave[i];
  if (kept) {
    gathered[int64_t(b) * maxb + pos] = kv.block_tables[int64_t(b) * maxb + blk];
    cnt[int64_t(b) * maxb + pos] = min(kBlock, n - kBlock * blk);
  }
  if (tid == 0 && (nb - 1) / 256 == int(blockIdx.x))
    num_kept[b] = s_prefix + s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
}

// The largest Local tile count: the sinks' blocks, the window's (one more when it is not
// block aligned), at most the block table's columns. A tile table row holds kTabHeader +
// this words.
int local_tiles_max(int sinks, int window, int max_blocks) {
  const int64_t t = int64_t((sinks + kBlock - 1) / kBlock) + (int64_t(window) + kBlock - 1) / kBlock + 1;
  return int(t < max_blocks ? t : max_blocks);
}

// One thread per (request, Local tile): the physical block of tile i of request b's Local
// view at its current length (word kTabHeader + i of its row; words 0-2: that length, the
// sinks and the window). Requests with an invalid length get the header only (the decode
// launch reports them).
__global__ __launch_bounds__(256) void local_tiles_kernel(sk_paged_kv kv, int sinks, int window, int row,
                                                          int32_t* __restrict__ tab) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int n = kv.seq_lens[b];
  int32_t* t = tab + int64_t(b) * row;
  if (i == 0) {
    t[0] = n;
    t[1] = sinks;
    t[2] = window;
  }
  if (n < 1 || n > kv.max_blocks * kBlock) return;
  DecodeParams P{};
  P.sinks = sinks;
  P.window = window;
  if (i >= request_tiles<kLocal>(P, b, n, 0)) return;
  int lo, hi;
  t[kTabHeader + i] = kv.block_tables[int64_t(b) * kv.max_blocks + local_tile(P, n, i, lo, hi)];
}

// Argument checks of every decode launch; the workspace is checked by the caller.
int check_decode(const float* q, const sk_paged_kv& kv, const void* k_new, const void* v_new, const float* out) {
  int st = check_kv(kv);
  if (st) return st;
  if (!q || !out) return SK_E_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return SK_E_NULL;
  return SK_OK;
}

// Enqueues one decode launch. scratch: a cleared workspace layout (header, tickets at
// kWsHeaderBytes, split partials at kPartialsOffset) of at least
// sk_workspace_bytes(batch, Hq) bytes; err: the device error word (may be null).
// The per-head q/k finish of a decode from a layer's raw q/k/v projection.
struct QKFinish {
  const uint16_t* g_q;
  const uint16_t* g_k;
  float eps;
  float rope_base;
};

template <int MODE, bool QK, bool HAS_SEL>
void launch_instance(bool single, int64_t grid, size_t lds, hipStream_t stream, const DecodeParams& P) {
  if (single)
    hipLaunchKernelGGL((decode_kernel<MODE, HAS_SEL, true, QK>), dim3(unsigned(grid)), dim3(kThreads), lds, stream, P);
  else
    hipLaunchKernelGGL((decode_kernel<MODE, HAS_SEL, false, QK>), dim3(unsigned(grid)), dim3(kThreads), lds, stream,
                       P);
}

// Batch launches: the balanced item order for ragged requests is a variant of its own
// (BAL), taken for batches above 64 requests; up to 64, the lengths are rarely ragged
// enough to pay for it (the variant's extra code measured 2-4 % slower on equal lengths).
template <int MODE, bool HAS_SEL>
void launch_batch(int64_t grid, size_t lds, hipStream_t stream, const DecodeParams& P) {
  if (P.kv.batch > 64)
    hipLaunchKernelGGL((decode_kernel<MODE, HAS_SEL, false, false, true>), dim3(unsigned(grid)), dim3(kThreads), lds,
                       stream, P);
  else
    hipLaunchKernelGGL((decode_kernel<MODE, HAS_SEL, false, false, false>), dim3(unsigned(grid)), dim3(kThreads), lds,
                       stream, P);
}

template <int MODE>
int enqueue_decode(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, int sinks, int window,
                   float scale, const int32_t* sel, int sel_value, const int32_t* lp, const int32_t* lc,
                   const int32_t* ln, float* out, uint8_t* scratch, int32_t* err, hipStream_t stream,
                   const int32_t* decl, int local_tokens, const QKFinish* qk = nullptr,
                   const int32_t* tab = nullptr) {
  DecodeParams P;
  P.q = q;
  P.kv = kv;
  P.k_new = reinterpret_cast<const uint16_t*>(k_new);
  P.v_new = reinterpret_cast<const uint16_t*>(v_new);
  P.sel = sel;
  P.sel_value = sel_value;
  P.list_phys = lp;
  P.list_cnt = lc;
  P.list_num = ln;
  P.out = out;
  P.err = err;
  P.tickets = reinterpret_cast<uint32_t*>(scratch + kWsHeaderBytes);
  P.partials = reinterpret_cast<float*>(scratch + kPartialsOffset);
  P.sinks = sinks;
  P.window = window;
  P.qscale = scale * kLog2e;
  P.decl = decl;
  P.local_tokens = local_tokens;
  P.g_q = qk ? qk->g_q : nullptr;
  P.g_k = qk ? qk->g_k : nullptr;
  P.qk_eps = qk ? qk->eps : 0.f;
  P.rope_base = qk ? qk->rope_base : 0.f;
  P.tab = tab;
  P.tab_tiles = local_tiles_max(sinks, window, kv.max_blocks);
  const int G = kv.num_q_heads / kv.num_kv_heads;
  // Grid: one workgroup per CU at most, fewer for small launches (an upper bound of the
  // work items from max_blocks), rounded to a multiple of the 8 XCDs.
  int64_t tiles_max = (MODE == kLocal)
                          ? int64_t((sinks + kBlock - 1) / kBlock) + (window + kBlock - 1) / kBlock + 1
                          : int64_t(kv.max_blocks);
  if (tiles_max > kv.max_blocks) tiles_max = kv.max_blocks;
  int64_t bound = int64_t(kv.batch) * kv.num_kv_heads * ((tiles_max + kMinTilesPerSplit - 1) / kMinTilesPerSplit);
  int64_t grid = bound < kGridCap ? bound : kGridCap;
  grid = (grid + 7) / 8 * 8;
  const int acc_region = std::max(kWavesPerWG * G * kHeadDim, 2 * kMaxSplits * G + 4 * kThreads);
  size_t lds = size_t(kThreads) * 16 + 128 * 4 + size_t(acc_region) * 4 + size_t(kWavesPerWG) * 16 * 4 * 2 +
               size_t(3 * kv.batch + 1 + 8 + (MODE == kViews ? kv.batch : 0)) * 4 +
               (kv.batch <= kOrderMaxBatch ? size_t(3 * kv.batch + 1) * 4 : 0);
  const bool single = kv.batch == 1 && grid >= 2 * int64_t(kv.num_kv_heads);
  if constexpr (MODE == kFull || MODE == kLocal) {
    if (qk) {
      if (sel)
        launch_instance<MODE, true, true>(single, grid, lds, stream, P);
      else
        launch_instance<MODE, true, false>(single, grid, lds, stream, P);
      return launch_status(hipGetLastError());
    }
  }
  if (qk) return SK_E_RANGE;  // the q/k finish exists for the Full and Local views
  if constexpr (MODE == kViews) {  // the views are the selector: always present; balanced order
    hipLaunchKernelGGL((decode_kernel<MODE, true, false, false, true>), dim3(unsigned(grid)), dim3(kThreads), lds,
                       stream, P);
  } else if (single) {
    if constexpr (MODE == kLocal) {
      if (tab) {  // descriptors from the step's tile table
        if (sel)
          hipLaunchKernelGGL((decode_kernel<MODE, true, true, false, false, true>), dim3(unsigned(grid)),
                             dim3(kThreads), lds, stream, P);
        else
          hipLaunchKernelGGL((decode_kernel<MODE, false, true, false, false, true>), dim3(unsigned(grid)),
                             dim3(kThreads), lds, stream, P);
        return launch_status(hipGetLastError());
      }
    }
    if (sel)
      hipLaunchKernelGGL((decode_kernel<MODE, true, true>), dim3(unsigned(grid)), dim3(kThreads), lds, stream, P);
    else
      hipLaunchKernelGGL((decode_kernel<MODE, false, true>), dim3(unsigned(grid)), dim3(kThreads), lds, stream, P);
  } else {
    if (sel)
      launch_batch<MODE, true>(grid, lds, stream, P);
    else
      launch_batch<MODE, false>(grid, lds, stream, P);
  }
  return launch_status(hipGetLastError());
}

template <int MODE>
int launch_decode(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, int sinks, int window,
                  float scale, const int32_t* sel, int sel_value, const int32_t* lp, const int32_t* lc,
                  const int32_t* ln, float* out, void* ws, size_t ws_bytes, hipStream_t stream,
                  const int32_t* decl = nullptr, int local_tokens = 0, const QKFinish* qk = nullptr,
                  const int32_t* tab = nullptr) {
  int st = check_decode(q, kv, k_new, v_new, out);
  if (st) return st;
  if (!ws) return SK_E_NULL;
  if (ws_bytes < sk_workspace_bytes(kv.batch, kv.num_q_heads)) return SK_E_WORKSPACE;
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  return enqueue_decode<MODE>(q, kv, k_new, v_new, sinks, window, scale, sel, sel_value, lp, lc, ln, out, base,
                              reinterpret_cast<int32_t*>(base), stream, decl, local_tokens, qk, tab);
}

int check_qk(const float* qkv, const uint16_t* g_q, const uint16_t* g_k, float eps, float rope_base) {
  if (!qkv || !g_q || !g_k) return SK_E_NULL;
  if (!(rope_base > 0.f) || !(eps >= 0.f)) return SK_E_RANGE;
  return SK_OK;
}

// ---- allocation-free Full view: the workspace lives in a file-scope device array
// (one copy per GPU, kept until the process ends). In host code `scratch` only names
// the symbol; its device address on the current GPU comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void scratch_clear_kernel(uint32_t* p, uint32_t words) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < words) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices];  // device address of `scratch` per GPU (null until set up)

// The scratch array's address on the current GPU; on the first call for that GPU, looks
// the address up and enqueues the clearing of its header and tickets on `stream`
// (a fill kernel, not a memset: the call may be captured in a graph).
int scratch_on_device(hipStream_t stream, uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_status(e);
  if (dev < 0 || dev >= kMaxDevices) return SK_E_RANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return launch_status(e);
    if (!ptr) return launch_status(hipErrorInvalidSymbol);
    const uint32_t words = uint32_t(kPartialsOffset / 4);
    hipLaunchKernelGGL(scratch_clear_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(ptr), words);
    e = hipGetLastError();
    if (e != hipSuccess) return launch_status(e);
    g_scratch[dev] = reinterpret_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return SK_OK;
}

}  // namespace
}  // namespace sk

using namespace sk;

extern "C" {

int oda_decode_local(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, int32_t sinks,
                     int32_t window, float scale, const int32_t* sel, int32_t sel_value, float* out, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (sinks < 0 || window < 1) return SK_E_RANGE;
  return launch_decode<kLocal>(q, kv, k_new, v_new, sinks, window, scale, sel, sel_value, nullptr, nullptr,
                               nullptr, out, ws, ws_bytes, stream);
}

size_t oda_local_tiles_bytes(int32_t batch, int32_t sinks, int32_t window, int32_t max_blocks) {
  if (batch < 1 || sinks < 0 || window < 1 || max_blocks < 1) return 0;
  return size_t(batch) * size_t(kTabHeader + local_tiles_max(sinks, window, max_blocks)) * 4;
}

int oda_local_tiles(sk_paged_kv kv, int32_t sinks, int32_t window, int32_t* tab, size_t tab_bytes,
                    hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!tab) return SK_E_NULL;
  if (sinks < 0 || window < 1) return SK_E_RANGE;
  if (tab_bytes < oda_local_tiles_bytes(kv.batch, sinks, window, kv.max_blocks)) return SK_E_WORKSPACE;
  const int row = kTabHeader + local_tiles_max(sinks, window, kv.max_blocks);
  hipLaunchKernelGGL(local_tiles_kernel, dim3(unsigned((row - kTabHeader + 255) / 256), unsigned(kv.batch)),
                     dim3(256), 0, stream, kv, sinks, window, row, tab);
  return launch_status(hipGetLastError());
}

int oda_decode_local_tiles(const float* q, sk_paged_kv kv, const int32_t* tab, size_t tab_bytes, const void* k_new,
                           const void* v_new, int32_t sinks, int32_t window, float scale, const int32_t* sel,
                           int32_t sel_value, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!tab) return SK_E_NULL;
  if (sinks < 0 || window < 1) return SK_E_RANGE;
  if (kv.batch >= 1 && kv.max_blocks >= 1 &&
      tab_bytes < oda_local_tiles_bytes(kv.batch, sinks, window, kv.max_blocks))
    return SK_E_WORKSPACE;
  return launch_decode<kLocal>(q, kv, k_new, v_new, sinks, window, scale, sel, sel_value, nullptr, nullptr,
                               nullptr, out, ws, ws_bytes, stream, nullptr, 0, nullptr, tab);
}

int oda_decode_full(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, float scale,
                    const int32_t* sel, int32_t sel_value, float* out, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return launch_decode<kFull>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, nullptr, nullptr, nullptr, out,
                              ws, ws_bytes, stream);
}

int oda_decode_local_qkv(const float* qkv, const uint16_t* g_q, const uint16_t* g_k, float eps, float rope_base,
                         sk_paged_kv kv, int32_t sinks, int32_t window, float scale, const int32_t* sel,
                         int32_t sel_value, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_qk(qkv, g_q, g_k, eps, rope_base);
  if (st) return st;
  if (sinks < 0 || window < 1) return SK_E_RANGE;
  const QKFinish qk{g_q, g_k, eps, rope_base};
  return launch_decode<kLocal>(qkv, kv, nullptr, nullptr, sinks, window, scale, sel, sel_value, nullptr, nullptr,
                               nullptr, out, ws, ws_bytes, stream, nullptr, 0, &qk);
}

int oda_decode_full_qkv(const float* qkv, const uint16_t* g_q, const uint16_t* g_k, float eps, float rope_base,
                        sk_paged_kv kv, float scale, const int32_t* sel, int32_t sel_value, float* out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  int st = check_qk(qkv, g_q, g_k, eps, rope_base);
  if (st) return st;
  const QKFinish qk{g_q, g_k, eps, rope_base};
  return launch_decode<kFull>(qkv, kv, nullptr, nullptr, 0, 1, scale, sel, sel_value, nullptr, nullptr, nullptr, out,
                              ws, ws_bytes, stream, nullptr, 0, &qk);
}

int oda_decode_full_noalloc(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, float scale,
                            const int32_t* sel, int32_t sel_value, float* out, int32_t* dev_err,
                            hipStream_t stream) {
  int st = check_decode(q, kv, k_new, v_new, out);
  if (st) return st;
  if (sk_workspace_bytes(kv.batch, kv.num_q_heads) > kScratchBytes) return SK_E_WORKSPACE;
  uint8_t* base = nullptr;
  st = scratch_on_device(stream, &base);
  if (st) return st;
  return enqueue_decode<kFull>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, nullptr, nullptr, nullptr, out, base,
                               dev_err, stream, nullptr, 0);
}

int da_decode_blocks(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new,
                     const uint32_t* keep_mask, int32_t* gathered, int32_t* gathered_cnt, int32_t* num_kept,
                     float scale, const int32_t* sel, int32_t sel_value, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!keep_mask || !gathered || !gathered_cnt || !num_kept || !ws) return SK_E_NULL;
  hipLaunchKernelGGL(gather_kernel, dim3(unsigned((kv.max_blocks + 255) / 256), unsigned(kv.batch)), dim3(256), 0,
                     stream, kv, keep_mask, sel, sel_value, gathered, gathered_cnt, num_kept,
                     reinterpret_cast<int32_t*>(ws));
  st = launch_status(hipGetLastError());
  if (st) return st;
  return launch_decode<kList>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, gathered, gathered_cnt, num_kept,
                              out, ws, ws_bytes, stream);
}

int da_gather(sk_paged_kv kv, const uint32_t* keep_mask, int32_t* gathered, int32_t* gathered_cnt, int32_t* num_kept,
              const int32_t* sel, int32_t sel_value, void* ws, hipStream_t stream) {
  int st = check_kv(kv);
  if (st) return st;
  if (!keep_mask || !gathered || !gathered_cnt || !num_kept) return SK_E_NULL;
  hipLaunchKernelGGL(gather_kernel, dim3(unsigned((kv.max_blocks + 255) / 256), unsigned(kv.batch)), dim3(256), 0,
                     stream, kv, keep_mask, sel, sel_value, gathered, gathered_cnt, num_kept,
                     reinterpret_cast<int32_t*>(ws));
  return launch_status(hipGetLastError());
}

int da_decode_declared(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, const int32_t* decl,
                       int32_t local_tokens, float scale, const int32_t* sel, int32_t sel_value, float* out,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!decl) return SK_E_NULL;
  if (local_tokens < 0) return SK_E_RANGE;
  return launch_decode<kDecl>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, nullptr, nullptr, nullptr, out, ws,
                              ws_bytes, stream, decl, local_tokens);
}

int da_decode_gathered(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, const int32_t* gathered,
                       const int32_t* gathered_cnt, const int32_t* num_kept, float scale, const int32_t* sel,
                       int32_t sel_value, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!gathered || !gathered_cnt || !num_kept) return SK_E_NULL;
  return launch_decode<kList>(q, kv, k_new, v_new, 0, 1, scale, sel, sel_value, gathered, gathered_cnt, num_kept,
                              out, ws, ws_bytes, stream);
}

int oda_decode_views(const float* q, sk_paged_kv kv, const void* k_new, const void* v_new, int32_t sinks,
                     int32_t window, float scale, const int32_t* view, const int32_t* gathered,
                     const int32_t* gathered_cnt, const int32_t* num_kept, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (!view || !gathered || !gathered_cnt || !num_kept) return SK_E_NULL;
  if (sinks < 0 || window < 1) return SK_E_RANGE;
  return launch_decode<kViews>(q, kv, k_new, v_new, sinks, window, scale, view, 0, gathered, gathered_cnt, num_kept,
                               out, ws, ws_bytes, stream);
}

}  // extern "C"
