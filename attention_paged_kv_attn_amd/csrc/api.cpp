// api.cpp — the C ABI of libpaged_attn: argument checks, workspace layout,
// the three launches (Assign -> split-K attention -> Combine) on the caller's
// stream, and optional per-launch event timing.  See include/paged_attn.h.
#include <hip/hip_runtime.h>
#include <cmath>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/paged_attn.h"
#include "pa_device.h"

namespace pa {
hipError_t launch_assign(const KParams& p, hipStream_t stream);
hipError_t launch_attention(const KParams& p, int kind, int grid, int paths, hipStream_t stream);
hipError_t launch_combine(const KParams& p, bool out_f32, int grid, hipStream_t stream);
hipError_t launch_static_begin(const KParams& p, hipStream_t stream);
}  // namespace pa

namespace {

thread_local int32_t g_last_hip_error = 0;

struct TimedCall {
  hipEvent_t ev[4];
};
std::mutex g_timing_mu;
bool g_timing = false;
std::vector<TimedCall> g_timed;

pa_status hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int32_t>(e);
  return PA_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int elt_size(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_F8E4M3: return 1;
    case PA_U8: return 1;
    default: return 0;
  }
}

pa_status default_workers(int32_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e);
  *out = 2 * cus;              // two persistent workgroups per compute unit
  return PA_OK;
}

pa_status check_params(const pa_params* p) {
  if (!p) return PA_ERR_INVALID_ARG;
  if (p->num_seqs < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->num_pages < 1 ||
      p->max_pages_per_seq < 1 || p->total_q < 0 || p->block_table_stride < p->max_pages_per_seq)
    return PA_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads) return PA_ERR_INVALID_ARG;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (128 % G) return PA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!is_pow2(p->page_size)) return PA_ERR_INVALID_ARG;
  if (p->window < 0 || p->landmark_chunk < 0) return PA_ERR_INVALID_ARG;
  if (p->block_mask_tile != 0 && (p->block_mask_tile < 64 || p->block_mask_tile % 64)) return PA_ERR_INVALID_ARG;
  if (p->num_workers < 0 || p->split_min_units < 0 || p->force_split_units < 0 || p->max_partial_slots < 0)
    return PA_ERR_INVALID_ARG;
  if (p->flags != 0) return PA_ERR_INVALID_ARG;
  if (p->split_mode != PA_SPLIT_DYNAMIC && p->split_mode != PA_SPLIT_STATIC) return PA_ERR_INVALID_ARG;
  if (p->static_splits < 0 || (p->split_mode == PA_SPLIT_STATIC && p->static_splits < 1)) return PA_ERR_INVALID_ARG;
  if (p->max_q_len < 0 || p->min_q_len < 0) return PA_ERR_INVALID_ARG;
  if (p->max_q_len > 0 && p->min_q_len > p->max_q_len) return PA_ERR_INVALID_ARG;
  if (p->pair_weight < 0 || p->pair_weight > 99) return PA_ERR_INVALID_ARG;
  if (p->fused_combine != 0 && p->fused_combine != 1) return PA_ERR_INVALID_ARG;
  if (p->qblock_per_kv_head != 0 && p->qblock_per_kv_head != 1) return PA_ERR_INVALID_ARG;
  if (!(p->softmax_scale > 0.f) || p->softmax_scale == INFINITY) return PA_ERR_INVALID_ARG;   // finite, positive
  return PA_OK;
}

// Which build of the attention kernel a call runs: without the prefill path
// when every Q-block is known to be small (a static split, or max_q_len * G
// <= 16), without the decode path when every one is known to be large
// (min_q_len * G > 16), else the general one.
int kernel_paths(const pa_params* p) {
  const int64_t G = p->num_q_heads / p->num_kv_heads;
  if (p->split_mode == PA_SPLIT_STATIC || (p->max_q_len > 0 && p->max_q_len * G <= pa::kSmallMaxRows))
    return 1;
  if (p->min_q_len * G > pa::kSmallMaxRows) return 2;
  return 0;
}

// Sequence Q-blocks (every query head of a sequence in one Q-block, units
// its (tile, kv head) pairs): a decode-only dynamic call whose kv heads split
// evenly over the four waves of a workgroup with each wave's query rows
// (hpw = Hkv / 4 heads x G x q_len) in one 16-row block.  A call with a block
// mask uses one Q-block per kv head instead (fwd_impl).
bool sequence_qblocks(const pa_params* p) {
  if (kernel_paths(p) != 1 || p->split_mode != PA_SPLIT_DYNAMIC || p->qblock_per_kv_head) return false;
  const int64_t G = p->num_q_heads / p->num_kv_heads;
  return p->num_kv_heads % 4 == 0 && p->max_q_len > 0 &&
         int64_t(p->max_q_len) * G * (p->num_kv_heads / 4) <= pa::kSmallMaxRows;
}

pa_status layout_of(const pa_params* p, pa_workspace_layout* L) {
  pa_status st = check_params(p);
  if (st != PA_OK) return st;
  int32_t P = p->num_workers;
  if (P == 0) {
    st = default_workers(&P);
    if (st != PA_OK) return st;
  }
  const int G = p->num_q_heads / p->num_kv_heads;
  const int64_t rows_large = (int64_t(p->total_q) * G + pa::kLargeRows - 1) / pa::kLargeRows;
  const int64_t n_qb_max = int64_t(p->num_kv_heads) * (p->num_seqs + rows_large);
  // P workers cut at most 2P Q-blocks (each range cuts its first and its
  // last); an odd P whose last worker pair is cut unevenly uses P + 1
  const int64_t max_slots = p->max_partial_slots ? p->max_partial_slots : 2 * (int64_t(P) + (P & 1));
  // a partial slot holds the largest Q-block the kernel build can meet
  int32_t slot_rows = kernel_paths(p) == 1 ? pa::kSmallMaxRows : pa::kLargeRows;
  if (sequence_qblocks(p)) slot_rows = std::max(slot_rows, p->max_q_len * p->num_q_heads);
  if (n_qb_max > (1 << 30) || max_slots > (1 << 24)) return PA_ERR_INVALID_ARG;
  std::memset(L, 0, sizeof(*L));
  size_t off = 0;
  L->header = off;        off = align256(off + pa::kHeaderInts * 4);
  L->seq_qb_base = off;   off = align256(off + size_t(p->num_seqs + 1) * 4);
  L->qb_desc = off;       off = align256(off + size_t(n_qb_max) * 32);
  L->unit_prefix = off;   off = align256(off + size_t(n_qb_max + 1) * 4);
  L->n_splits = off;      off = align256(off + size_t(n_qb_max) * 4);
  L->slot_base = off;     off = align256(off + size_t(n_qb_max) * 4);
  L->combine_list = off;  off = align256(off + size_t(n_qb_max) * 4);
  L->done = off;          off = align256(off + size_t(n_qb_max) * 4);
  L->partial_lse = off;   off = align256(off + size_t(max_slots) * slot_rows * 4);
  L->partial_o = off;     off = align256(off + size_t(max_slots) * slot_rows * p->head_dim * 4);
  L->total = off;
  L->n_qb_max = int32_t(n_qb_max);
  L->max_slots = int32_t(max_slots);
  L->num_workers = P;
  L->slot_rows = slot_rows;
  L->qblock_heads = sequence_qblocks(p) ? p->num_q_heads : G;
  return PA_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// A device tensor of the given rank/dtype whose innermost stride is 1 and whose
// rows start on 16-byte boundaries.
pa_status check_tensor(const pa_tensor* t, int rank, int dtype, bool rows16) {
  if (!t || !t->data) return PA_ERR_INVALID_ARG;
  if (t->rank != rank) return PA_ERR_INVALID_ARG;
  if (t->dtype != dtype) return PA_ERR_UNSUPPORTED;
  for (int i = 0; i < rank; ++i)
    if (t->shape[i] < 0) return PA_ERR_INVALID_ARG;
  if (rank > 1 && t->stride[rank - 1] != 1) return PA_ERR_UNSUPPORTED;
  if (rows16) {
    const int es = elt_size(dtype);
    if (!aligned16(t->data)) return PA_ERR_INVALID_ARG;
    for (int i = 0; i < rank - 1; ++i)
      if ((t->stride[i] * es) % 16) return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

// The launches of one call on `stream`: Assign (or the static split's
// header reset), the attention kernel, and Combine unless it is fused or the
// static split has one split per Q-block.  ev, when given, receives an event
// before each launch and one after the last.
hipError_t launch_all(const pa::KParams& kp, const pa_params& P, const pa_workspace_layout& L, int kind,
                      int paths, hipStream_t stream, hipEvent_t* ev) {
  const bool is_static = P.split_mode == PA_SPLIT_STATIC;
  const int64_t n_static_qb = int64_t(P.num_seqs) * P.num_kv_heads;
  hipError_t e;
  if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess) return e;
  e = is_static ? pa::launch_static_begin(kp, stream) : pa::launch_assign(kp, stream);
  if (e != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[1], stream)) != hipSuccess) return e;
  const int64_t n_items = n_static_qb * P.static_splits;
  const int grid = is_static ? static_cast<int>(std::min<int64_t>(n_items, L.num_workers)) : L.num_workers;
  e = pa::launch_attention(kp, kind, grid, paths, stream);
  if (e != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[2], stream)) != hipSuccess) return e;
  if (!P.fused_combine && (!is_static || P.static_splits > 1)) {
    const int cgrid = is_static ? static_cast<int>(std::min<int64_t>(n_static_qb, L.num_workers)) : L.num_workers;
    e = pa::launch_combine(kp, kind == pa::KIND_F32, cgrid, stream);
    if (e != hipSuccess) return e;
  }
  if (ev && (e = hipEventRecord(ev[3], stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* paged_attn_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_SCRATCH: return "problem needs more workspace than the no-allocation entry point holds";
  }
  return "unknown status";
}

int32_t paged_attn_last_hip_error(void) { return g_last_hip_error; }

pa_status paged_attn_workspace_layout(const pa_params* params, pa_workspace_layout* layout) {
  if (!layout) return PA_ERR_INVALID_ARG;
  return layout_of(params, layout);
}

pa_status paged_attn_workspace_size(const pa_params* params, size_t* bytes) {
  if (!bytes) return PA_ERR_INVALID_ARG;
  pa_workspace_layout L;
  pa_status st = layout_of(params, &L);
  if (st == PA_OK) *bytes = L.total;
  return st;
}

pa_status paged_attn_device_info(int32_t device, pa_device_info* info) {
  if (!info) return PA_ERR_INVALID_ARG;
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_fail(e);
  std::memset(info, 0, sizeof(*info));
  info->compute_units = prop.multiProcessorCount;
  info->lds_bytes_per_workgroup = static_cast<int32_t>(prop.sharedMemPerBlock);
  info->default_workers = 2 * prop.multiProcessorCount;
  std::strncpy(info->arch, prop.gcnArchName, sizeof(info->arch) - 1);
  return PA_OK;
}

pa_status paged_attn_plan_split(const pa_params* p, const int32_t* seq_lens_h, const int32_t* qsl_h,
                                int32_t has_block_mask, int32_t* split_mode, int32_t* static_splits) {
  if (!split_mode || !static_splits || !seq_lens_h || !qsl_h) return PA_ERR_INVALID_ARG;
  pa_workspace_layout L;
  pa_status st = layout_of(p, &L);
  if (st != PA_OK) return st;
  *split_mode = PA_SPLIT_DYNAMIC;
  *static_splits = 0;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int64_t Pw = L.num_workers;
  const int64_t L_min = p->split_min_units ? p->split_min_units : 8;
  int64_t U = 0, T_max = 0, n_qb = int64_t(p->num_seqs) * p->num_kv_heads;
  for (int b = 0; b < p->num_seqs; ++b) {
    const int ql = qsl_h[b + 1] - qsl_h[b], ctx = seq_lens_h[b];
    if (ql < 0 || ql > ctx) return PA_ERR_INVALID_ARG;
    if (ql == 0) continue;
    if (int64_t(ql) * G > pa::kSmallMaxRows) return PA_OK;      // static holds small Q-blocks only
    // the Q-block's tiles, as the device counts them (positions ctx - ql .. ctx - 1)
    const int hi = ctx - 1;
    int lo = 0;
    if (p->window > 0) {
      lo = std::max(0, ctx - ql - p->window + 1);
      if (p->window_expand_to_chunk && p->landmark_chunk > 0) lo = (lo / p->landmark_chunk) * p->landmark_chunk;
    }
    const int64_t n = hi >= lo ? hi / pa::kUnitKeys - lo / pa::kUnitKeys + 1 : 0;
    U += n * p->num_kv_heads;
    T_max = std::max(T_max, n);
  }
  if (has_block_mask || U == 0) return PA_OK;
  // the busiest worker's tiles under the dynamic task map, plus Assign and Combine
  const int64_t dyn = std::max(L_min, (U + Pw - 1) / Pw) + PA_POLICY_ASSIGN_UNITS + PA_POLICY_COMBINE_UNITS;
  int64_t best = -1, best_S = 0;
  const int64_t S_cap = std::max<int64_t>(1, (T_max + L_min - 1) / L_min);
  for (int64_t S = 1; S <= S_cap; ++S) {
    if (S > 1 && n_qb * S > L.max_slots) break;
    const int64_t rounds = (n_qb * S + Pw - 1) / Pw;
    const int64_t cost = rounds * ((T_max + S - 1) / S) + (S > 1 ? PA_POLICY_COMBINE_UNITS : 0);
    if (best < 0 || cost < best) {
      best = cost;
      best_S = S;
    }
  }
  if (best >= 0 && best <= dyn) {
    *split_mode = PA_SPLIT_STATIC;
    *static_splits = static_cast<int32_t>(best_S);
  }
  return PA_OK;
}

pa_status paged_attn_validate_host(const pa_params* p, const int32_t* seq_lens_h, const int32_t* qsl_h,
                                   const int32_t* bt_h, const uint8_t* mask_h, int32_t mask_heads,
                                   int32_t mask_q_tiles, int32_t mask_k_tiles) {
  pa_status st = check_params(p);
  if (st != PA_OK) return st;
  if (!seq_lens_h || !qsl_h || !bt_h) return PA_ERR_INVALID_ARG;
  if (qsl_h[0] != 0 || qsl_h[p->num_seqs] != p->total_q) return PA_ERR_INVALID_ARG;
  const int tile = p->block_mask_tile ? p->block_mask_tile : 128;
  for (int b = 0; b < p->num_seqs; ++b) {
    const int ql = qsl_h[b + 1] - qsl_h[b];
    const int ctx = seq_lens_h[b];
    if (ql < 0 || ctx < 0 || ql > ctx) return PA_ERR_INVALID_ARG;
    const int64_t pages = (int64_t(ctx) + p->page_size - 1) / p->page_size;
    if (pages > p->max_pages_per_seq) return PA_ERR_INVALID_ARG;
    for (int64_t i = 0; i < pages; ++i) {
      const int32_t pg = bt_h[int64_t(b) * p->block_table_stride + i];
      if (pg < 0 || pg >= p->num_pages) return PA_ERR_INVALID_ARG;
    }
    if (mask_h) {
      if (mask_heads != 1 && mask_heads != p->num_q_heads) return PA_ERR_INVALID_ARG;
      if (ctx > int64_t(mask_q_tiles) * tile || ctx > int64_t(mask_k_tiles) * tile) return PA_ERR_INVALID_ARG;
    }
  }
  return PA_OK;
}

pa_status paged_attn_kernel_timing(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing = enable != 0;
  return PA_OK;
}

pa_status paged_attn_kernel_timing_read(float* ms_assign, float* ms_attention, float* ms_combine,
                                        int32_t* calls) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  float a = 0, b = 0, c = 0;
  pa_status st = PA_OK;
  for (auto& t : g_timed) {
    hipError_t e = hipEventSynchronize(t.ev[3]);
    float x = 0, y = 0, z = 0;
    if (e == hipSuccess) e = hipEventElapsedTime(&x, t.ev[0], t.ev[1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&y, t.ev[1], t.ev[2]);
    if (e == hipSuccess) e = hipEventElapsedTime(&z, t.ev[2], t.ev[3]);
    if (e != hipSuccess) st = hip_fail(e);
    a += x; b += y; c += z;
    for (auto& ev : t.ev) (void)hipEventDestroy(ev);
  }
  if (calls) *calls = static_cast<int32_t>(g_timed.size());
  g_timed.clear();
  if (ms_assign) *ms_assign = a;
  if (ms_attention) *ms_attention = b;
  if (ms_combine) *ms_combine = c;
  return st;
}

}  // extern "C"

namespace {

// The whole call on a given workspace.  from_scratch: the workspace is the
// library's own scratch array (the no-allocation entry point), which reports a
// problem too large for it as PA_ERR_SCRATCH and records no timing events.
pa_status fwd_impl(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                   const int32_t* block_table, const int32_t* seq_lens, const int32_t* query_start_loc,
                   const pa_tensor* block_mask, const pa_scales* scales, pa_tensor* out, pa_tensor* lse,
                   const pa_params* params, void* workspace, size_t workspace_bytes, void* stream_ptr,
                   bool from_scratch) {
  pa_workspace_layout L;
  pa_status st = layout_of(params, &L);
  if (st != PA_OK) return st;
  const pa_params& P = *params;
  if (!q || !k_cache || !v_cache || !out || !lse) return PA_ERR_INVALID_ARG;
  const int dt = q->dtype;
  if (dt != PA_F32 && dt != PA_BF16 && dt != PA_F8E4M3) return PA_ERR_UNSUPPORTED;
  if ((st = check_tensor(q, 3, dt, true)) != PA_OK) return st;
  if ((st = check_tensor(k_cache, 4, dt, true)) != PA_OK) return st;
  if ((st = check_tensor(v_cache, 4, dt, true)) != PA_OK) return st;
  const int out_dt = dt == PA_F32 ? PA_F32 : PA_BF16;
  if ((st = check_tensor(out, 3, out_dt, true)) != PA_OK) return st;
  if (!lse || !lse->data || lse->rank != 2) return PA_ERR_INVALID_ARG;
  if (lse->dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (!block_table || !seq_lens || !query_start_loc) return PA_ERR_INVALID_ARG;
  const int64_t d = P.head_dim;
  if (q->shape[0] != P.total_q || q->shape[1] != P.num_q_heads || q->shape[2] != d) return PA_ERR_INVALID_ARG;
  for (const pa_tensor* c : {k_cache, v_cache})
    if (c->shape[0] != P.num_pages || c->shape[1] != P.page_size || c->shape[2] != P.num_kv_heads ||
        c->shape[3] != d)
      return PA_ERR_INVALID_ARG;
  if (out->shape[0] != P.total_q || out->shape[1] != P.num_q_heads || out->shape[2] != d) return PA_ERR_INVALID_ARG;
  if (lse->shape[0] != P.total_q || lse->shape[1] != P.num_q_heads) return PA_ERR_INVALID_ARG;
  if (block_mask) {
    if ((st = check_tensor(block_mask, 4, PA_U8, false)) != PA_OK) return st;
    if (block_mask->shape[0] != P.num_seqs ||
        (block_mask->shape[1] != 1 && block_mask->shape[1] != P.num_q_heads) ||
        block_mask->shape[2] < 1 || block_mask->shape[3] < 1)
      return PA_ERR_INVALID_ARG;
  }
  int scale_mode = 0;
  if (dt == PA_F8E4M3) {
    if (!scales || !scales->q_scale || !scales->k_scale || !scales->v_scale) return PA_ERR_INVALID_ARG;
    const int kv_mode = scales->mode & ~PA_SCALE_Q_PER_TOKEN_HEAD;
    if (kv_mode != PA_SCALE_PER_TENSOR && kv_mode != PA_SCALE_PER_PAGE_HEAD) return PA_ERR_INVALID_ARG;
    if (kv_mode == PA_SCALE_PER_PAGE_HEAD && P.page_size < 64) return PA_ERR_UNSUPPORTED;
    scale_mode = scales->mode;
  }
  const bool is_static = P.split_mode == PA_SPLIT_STATIC;
  const int64_t n_static_qb = int64_t(P.num_seqs) * P.num_kv_heads;
  if (is_static) {
    if (block_mask) return PA_ERR_UNSUPPORTED;
    if (P.static_splits > 1 && n_static_qb * P.static_splits > L.max_slots) return PA_ERR_INVALID_ARG;
    if (n_static_qb * P.static_splits > (1 << 30)) return PA_ERR_INVALID_ARG;
  }
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255)) return PA_ERR_WORKSPACE;
  if (workspace_bytes < L.total) return from_scratch ? PA_ERR_SCRATCH : PA_ERR_WORKSPACE;
  if (P.total_q == 0) return PA_OK;

  pa::KParams kp;
  std::memset(&kp, 0, sizeof(kp));
  kp.q = q->data; kp.q_st = q->stride[0]; kp.q_sh = q->stride[1];
  kp.k = k_cache->data; kp.k_sp = k_cache->stride[0]; kp.k_ss = k_cache->stride[1]; kp.k_sh = k_cache->stride[2];
  kp.v = v_cache->data; kp.v_sp = v_cache->stride[0]; kp.v_ss = v_cache->stride[1]; kp.v_sh = v_cache->stride[2];
  kp.out = out->data; kp.o_st = out->stride[0]; kp.o_sh = out->stride[1];
  kp.lse = static_cast<float*>(lse->data); kp.l_st = lse->stride[0]; kp.l_sh = lse->stride[1];
  kp.bt = block_table; kp.bt_stride = P.block_table_stride;
  kp.seq_lens = seq_lens; kp.qsl = query_start_loc;
  if (block_mask) {
    kp.bm = static_cast<const uint8_t*>(block_mask->data);
    kp.bm_sb = block_mask->stride[0]; kp.bm_sh = block_mask->stride[1];
    kp.bm_sq = block_mask->stride[2]; kp.bm_sk = block_mask->stride[3];
    kp.bm_heads = static_cast<int32_t>(block_mask->shape[1]);
    kp.bm_nq = static_cast<int32_t>(block_mask->shape[2]);
    kp.bm_nk = static_cast<int32_t>(block_mask->shape[3]);
  }
  kp.bm_tile = P.block_mask_tile ? P.block_mask_tile : 128;
  if (scale_mode) {
    kp.q_scale = scales->q_scale; kp.k_scale = scales->k_scale; kp.v_scale = scales->v_scale;
  }
  kp.scale_mode = scale_mode;
  kp.B = P.num_seqs; kp.Hq = P.num_q_heads; kp.Hkv = P.num_kv_heads; kp.G = P.num_q_heads / P.num_kv_heads;
  kp.D = P.head_dim; kp.page_size = P.page_size;
  kp.page_shift = __builtin_ctz(static_cast<unsigned>(P.page_size));
  kp.num_pages = P.num_pages; kp.total_q = P.total_q; kp.max_pages = P.max_pages_per_seq;
  kp.sm_log2 = P.softmax_scale * 1.4426950408889634f;
  kp.causal = P.causal ? 1 : 0;
  kp.window = P.window;
  kp.expand = P.window_expand_to_chunk ? 1 : 0;
  kp.landmark = P.landmark_chunk;
  kp.P = L.num_workers;
  kp.L_min = P.split_min_units ? P.split_min_units : 8;
  kp.force_L = P.force_split_units;
  kp.max_slots = L.max_slots;
  kp.n_qb_max = L.n_qb_max;
  kp.static_S = is_static ? P.static_splits : 0;
  kp.max_q_len = P.max_q_len;
  kp.min_q_len = P.min_q_len;
  const int paths = kernel_paths(params);
  kp.pair_w = P.pair_weight ? P.pair_weight : (paths == 1 ? PA_PAIR_WEIGHT_SMALL : PA_PAIR_WEIGHT_GENERAL);
  kp.fused = P.fused_combine ? 1 : 0;
  kp.slot_rows = L.slot_rows;
  // with a block mask the units of a Q-block follow the mask per kv head
  kp.seq_qb = sequence_qblocks(params) && !block_mask ? 1 : 0;
  kp.qbh = kp.seq_qb ? P.num_q_heads : kp.G;
  char* ws = static_cast<char*>(workspace);
  kp.hdr = reinterpret_cast<int32_t*>(ws + L.header);
  kp.seq_qb_base = reinterpret_cast<int32_t*>(ws + L.seq_qb_base);
  kp.qb_desc = reinterpret_cast<int32_t*>(ws + L.qb_desc);
  kp.unit_prefix = reinterpret_cast<int32_t*>(ws + L.unit_prefix);
  kp.n_splits = reinterpret_cast<int32_t*>(ws + L.n_splits);
  kp.slot_base = reinterpret_cast<int32_t*>(ws + L.slot_base);
  kp.combine_list = reinterpret_cast<int32_t*>(ws + L.combine_list);
  kp.done = reinterpret_cast<int32_t*>(ws + L.done);
  kp.part_lse = reinterpret_cast<float*>(ws + L.partial_lse);
  kp.part_o = reinterpret_cast<float*>(ws + L.partial_o);

  const int kind = dt == PA_F32 ? pa::KIND_F32 : dt == PA_BF16 ? pa::KIND_BF16 : pa::KIND_F8;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);

  TimedCall tc;
  int n_events = 0;
  bool timing = false;
  if (!from_scratch) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    timing = g_timing;
  }
  // events of a call that fails are destroyed here; a HIP failure after the
  // first launch leaves the launches before it enqueued
  auto fail = [&](hipError_t e) {
    for (int i = 0; i < n_events; ++i) (void)hipEventDestroy(tc.ev[i]);
    return hip_fail(e);
  };
  if (timing) {
    for (auto& ev : tc.ev) {
      hipError_t e = hipEventCreate(&ev);
      if (e != hipSuccess) return fail(e);
      ++n_events;
    }
  }
  // sequence Q-blocks run a kernel build of their own
  hipError_t e = launch_all(kp, P, L, kind, kp.seq_qb ? 3 : paths, stream, timing ? tc.ev : nullptr);
  if (e != hipSuccess) return fail(e);
  if (timing) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timed.push_back(tc);
  }
  return PA_OK;
}

// The library's own workspace for callers that cannot allocate.  In host code
// the name stands for the array only symbolically; its device address (one
// copy per device) comes from hipGetSymbolAddress, once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

// The scratch array's address on the current device (looked up on the first
// call there, with that device current, and kept).
pa_status scratch_on_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status paged_attn_fwd(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* query_start_loc, const pa_tensor* block_mask,
                         const pa_scales* scales, pa_tensor* out, pa_tensor* lse,
                         const pa_params* params, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return fwd_impl(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, block_mask, scales, out, lse,
                  params, workspace, workspace_bytes, stream, false);
}

pa_status paged_attn_fwd_noalloc(const pa_tensor* q, const pa_tensor* k_cache, const pa_tensor* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* query_start_loc, const pa_tensor* block_mask,
                                 const pa_scales* scales, pa_tensor* out, pa_tensor* lse,
                                 const pa_params* params, void* stream) {
  void* ws = nullptr;
  const pa_status st = scratch_on_current_device(&ws);
  if (st != PA_OK) return st;
  return fwd_impl(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, block_mask, scales, out, lse,
                  params, ws, PA_NOALLOC_SCRATCH_BYTES, stream, true);
}

}  // extern "C"
