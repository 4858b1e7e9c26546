// pa_device.h — kernel parameter block and the integer rules of the work split,
// shared by the Assign, attention and Combine kernels of libpaged_attn.
//
// The split follows "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2
// (Assign cuts every KV sequence into tiles and balances the tiles over
// persistent workgroups; Split-K emits partial output + LSE; Combine merges
// them) and §3.3 (pick the chunk length from the total load, then cut each
// request by its real KV length; a task owned by one workgroup writes its
// result directly), with the Q-block grouping of "vLLM Triton Attention
// Backend Deep Dive", §3 (all query heads of one KV head, several tokens).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kUnitKeys = 64;        // keys per unit (one KV tile)
constexpr int kSmallMaxRows = 16;    // q_len * G <= 16: one Q-block holds all query tokens of (b, g)
constexpr int kLargeRows = 128;      // otherwise Q-blocks of 128 / G tokens
constexpr int kThreads = 256;        // four wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kHeaderInts = 16;
constexpr int kMaskListCap = 1024;   // active-tile list entries kept in LDS at once

enum HeaderField {
  H_U = 0, H_P = 1, H_L = 2, H_NQB = 3, H_NSLOTS = 4, H_NCOMBINE = 5, H_NWORKERS = 6,
  H_ERROR = 7, H_MAXSLOTS = 8, H_L0 = 9
};

enum DevError { E_NONE = 0, E_QSL = 1, E_QLEN = 2, E_SLOTS = 3, E_PAGE = 5, E_STATIC_ROWS = 6, E_QLEN_HINT = 7 };

enum Kind { KIND_F32 = 0, KIND_BF16 = 1, KIND_F8 = 2 };

struct KParams {
  // inputs (element strides)
  const void* q;  int64_t q_st, q_sh;
  const void* k;  int64_t k_sp, k_ss, k_sh;
  const void* v;  int64_t v_sp, v_ss, v_sh;
  void* out;      int64_t o_st, o_sh;
  float* lse;     int64_t l_st, l_sh;
  const int32_t* bt; int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  const uint8_t* bm; int64_t bm_sb, bm_sh, bm_sq, bm_sk;
  int32_t bm_heads, bm_nq, bm_nk, bm_tile;
  const float* q_scale; const float* k_scale; const float* v_scale;
  int32_t scale_mode;   // bits 0-1: K/V scale kind (1 per tensor, 2 per (page, kv head)); bit 2: Q per (token, head)
  // sizes
  int32_t B, Hq, Hkv, G, D, page_size, page_shift, num_pages, total_q, max_pages;
  // scores and masks
  float sm_log2;     // softmax_scale * log2(e)
  int32_t causal, window, expand, landmark;
  // split
  int32_t P, L_min, force_L, max_slots, n_qb_max;
  int32_t static_S;  // > 0: static split, every Q-block cut into static_S equal tile ranges (no task map)
  int32_t max_q_len; // > 0: the caller's bound on every q_len (checked by Assign)
  int32_t min_q_len; // > 0: the caller's bound below every non-zero q_len (checked by Assign)
  int32_t pair_w;    // percent of a worker pair's 2L units given to its first worker
  int32_t fused;     // 1: the last workgroup to finish a split Q-block merges it (no Combine launch)
  int32_t slot_rows; // rows per partial slot: the kernel build's largest Q-block
  int32_t seq_qb;    // 1: one Q-block per sequence with all its query heads (decode, heads interleaved)
  int32_t qbh;       // query heads per token in a Q-block's rows: Hq when seq_qb, else G
  // workspace
  int32_t* hdr; int32_t* seq_qb_base; int32_t* qb_desc; int32_t* unit_prefix;
  int32_t* n_splits; int32_t* slot_base; int32_t* combine_list;
  int32_t* done;     // per Q-block: split pieces finished (fused combine)
  float* part_lse; float* part_o;
};

// First key a query at `pos` may see under the sliding window.
__device__ __forceinline__ int window_left(const KParams& p, int pos) {
  int left = pos - p.window + 1;
  if (left < 0) left = 0;
  if (p.expand && p.landmark > 0) left = (left / p.landmark) * p.landmark;
  return left;
}

// 64-key tile range [t_lo, t_hi] a Q-block with positions pos_lo..pos_hi may
// touch; false when it touches none.
__device__ __forceinline__ bool qblock_tiles(const KParams& p, int ctx, int pos_lo, int pos_hi,
                                             int& t_lo, int& t_hi) {
  int hi = p.causal ? min(ctx - 1, pos_hi) : ctx - 1;
  int lo = p.window > 0 ? window_left(p, pos_lo) : 0;
  if (hi < lo) return false;
  t_lo = lo / kUnitKeys;
  t_hi = hi / kUnitKeys;
  return true;
}

// Block-mask test of a 64-key tile for a Q-block: set for some query tile
// covering pos_lo..pos_hi and some query head of kv head g.
__device__ __forceinline__ bool mask_union(const KParams& p, int b, int g, int pos_lo, int pos_hi,
                                           int tile) {
  const int kt = (tile * kUnitKeys) / p.bm_tile;
  if (kt >= p.bm_nk) return false;
  const int qt0 = pos_lo / p.bm_tile;
  int qt1 = pos_hi / p.bm_tile;
  if (qt1 >= p.bm_nq) qt1 = p.bm_nq - 1;
  const int h0 = p.bm_heads == 1 ? 0 : g * p.G;
  const int h1 = p.bm_heads == 1 ? 1 : (g + 1) * p.G;
  const uint8_t* base = p.bm + b * p.bm_sb + kt * p.bm_sk;
  for (int hm = h0; hm < h1; ++hm)
    for (int qt = qt0; qt <= qt1; ++qt)
      if (base[hm * p.bm_sh + qt * p.bm_sq]) return true;
  return false;
}

// The workers' unit ranges: pairs (2k, 2k + 1) share 2L units, the first
// L0 to worker 2k (L0 = L is the even split).
struct WorkerMap {
  int L, L0;
  __device__ __forceinline__ static int first_len(int L, int pair_w) {
    const int Lp = 2 * L;
    return min(max((Lp * pair_w + 50) / 100, 1), Lp - 1);
  }
  __device__ __forceinline__ int worker_of(int u) const {
    const int Lp = 2 * L;
    const int k = u / Lp;
    return 2 * k + (u - k * Lp >= L0 ? 1 : 0);
  }
  __device__ __forceinline__ int start(int w) const { return (w >> 1) * 2 * L + (w & 1) * L0; }
  __device__ __forceinline__ int size(int w) const { return (w & 1) ? 2 * L - L0 : L0; }
};

// Decoded Q-block: rows are (token t0 + r / qbh, head g * G + r % qbh), with
// qbh = G (one kv head) or Hq (a sequence Q-block, g = 0).
struct QBlock {
  int b, g, t0, nt, rows, ql, ctx, q0, pos_lo, pos_hi;
};

// The descriptor is 8 ints: b, g, t0, nt, then the sequence's q0, q_len and
// seq_len (copied by Assign so one scalar load brings everything).
__device__ __forceinline__ QBlock load_qblock(const KParams& p, int q) {
  QBlock x;
  // scalar loads: the descriptor is the same for the whole wave, and a scalar
  // load does not wait on the wave's vector loads in flight
  typedef int cint __attribute__((address_space(4)));
  const cint* dp = (const cint*)(p.qb_desc + 8 * (int64_t)q);
  x.b = dp[0];
  x.g = dp[1];
  x.t0 = dp[2];
  x.nt = dp[3];
  x.rows = x.nt * p.qbh;
  x.q0 = dp[4];
  x.ql = dp[5];
  x.ctx = dp[6];
  x.pos_lo = x.ctx - x.ql + x.t0;
  x.pos_hi = x.pos_lo + x.nt - 1;
  return x;
}

// Static split (no task map): Q-block q is (b = q / Hkv, g = q % Hkv) and
// holds every query token of (b, g), so each sequence needs q_len * G <= 16.
// Reads the sequence's metadata directly; returns E_NONE or the error found.
__device__ __forceinline__ int static_qblock(const KParams& p, int q, QBlock& x) {
  const int b = q / p.Hkv;
  const int q0 = p.qsl[b], q1 = p.qsl[b + 1];
  x.b = b;
  x.g = q - b * p.Hkv;
  x.t0 = 0;
  x.q0 = q0;
  x.ql = q1 - q0;
  x.nt = x.ql;
  x.rows = x.ql * p.G;
  x.ctx = p.seq_lens[b];
  x.pos_lo = x.ctx - x.ql;
  x.pos_hi = x.ctx - 1;
  if (q0 < 0 || x.ql < 0 || q1 > p.total_q) return E_QSL;
  if (x.ql > x.ctx) return E_QLEN;
  if (x.rows > kSmallMaxRows) return E_STATIC_ROWS;
  return E_NONE;
}

// The tiles t_lo .. t_lo + n - 1 of a static Q-block, cut into runs of
// c = ceil(n / S) tiles; split s owns [s c, min(n, (s + 1) c)) and the ns
// non-empty splits are 0 .. ns - 1.
struct StaticSplit {
  int t_lo, n, c, ns;
};

__device__ __forceinline__ StaticSplit static_split(const KParams& p, const QBlock& x) {
  StaticSplit sp{0, 0, 1, 0};
  int t_hi = 0;
  if (x.ql > 0 && qblock_tiles(p, x.ctx, x.pos_lo, x.pos_hi, sp.t_lo, t_hi)) {
    sp.n = t_hi - sp.t_lo + 1;
    sp.c = (sp.n + p.static_S - 1) / p.static_S;
    sp.ns = (sp.n + sp.c - 1) / sp.c;
  }
  return sp;
}

}  // namespace pa
