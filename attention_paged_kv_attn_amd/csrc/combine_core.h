// combine_core.h — the LSE-weighted merge of a split Q-block's partials,
// used by the Combine kernel and by the attention kernel's fused combine.
//
// "Triton-TLE rewrite of Tencent HPC-Ops Attention", §1.2: Combine
// re-normalises the partial outputs of the KV chunks by their LSE, which is
// mathematically the same as full attention; §3.3 gives the same merge on raw
// online-softmax states.  For every row of a split Q-block:
//   M = max_s LSE_s;  LSE = M + ln sum_s exp(LSE_s - M);  O = sum_s exp(LSE_s - LSE) O_s.
// Parts with LSE_s = -inf weigh 0; a row whose parts are all -inf (or a
// Q-block with no unit at all) gets O = 0 and LSE = -inf.
#pragma once

#include "pa_device.h"

namespace pa {

typedef float f32x4c __attribute__((ext_vector_type(4)));
typedef unsigned u32x4c __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned pack_bf16x2_c(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// Partials cross compute units (and XCDs, whose L2s are not coherent with one
// another) inside one kernel when the merge is fused: they are written and
// read with device-coherent accesses (relaxed agent-scope atomics), which go
// past the XCD's L2, so no cache write-back or invalidation is needed.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One split merged into a running (m, z, o) state (natural-log domain LSEs):
// m = running max, z = sum of e^(LSE_s - m), o = sum of e^(LSE_s - m) O_s.
struct MergeState {
  float m, z, o[8];
};

// A split's 8 output values of a row (already loaded) merged into st.  An
// empty part (LSE = -inf, O written as 0) weighs nothing.
__device__ __forceinline__ void merge_part(MergeState& st, float ls, const f32x4c& a, const f32x4c& b) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (!(ls > -__builtin_huge_valf())) return;
  // explicit fused multiply-adds: every caller (the Combine kernel, the fused
  // merge) rounds alike, whatever contraction the compiler would choose
  const float m_new = fmaxf(st.m, ls);
  const float alpha = st.m == -__builtin_huge_valf() ? 0.f : exp2f((st.m - m_new) * kLog2e);
  const float w = exp2f((ls - m_new) * kLog2e);
  st.z = __builtin_fmaf(st.z, alpha, w);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    st.o[k] = __builtin_fmaf(w, a[k], st.o[k] * alpha);
    st.o[4 + k] = __builtin_fmaf(w, b[k], st.o[4 + k] * alpha);
  }
  st.m = m_new;
}

template <bool COHERENT>
__device__ __forceinline__ void load_part(const float* lp, const float* src, float& ls, f32x4c& a, f32x4c& b) {
  if constexpr (COHERENT) {
    ls = load_coherent(lp);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = load_coherent(src + k);
      b[k] = load_coherent(src + 4 + k);
    }
  } else {
    ls = *lp;
    a = *reinterpret_cast<const f32x4c*>(src);
    b = *reinterpret_cast<const f32x4c*>(src + 4);
  }
}

__device__ __forceinline__ void merge_state(MergeState& st, const MergeState& other) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (other.m == -__builtin_huge_valf()) return;
  const float m_new = fmaxf(st.m, other.m);
  const float a = st.m == -__builtin_huge_valf() ? 0.f : exp2f((st.m - m_new) * kLog2e);
  const float b = exp2f((other.m - m_new) * kLog2e);
  st.z = __builtin_fmaf(st.z, a, other.z * b);
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = __builtin_fmaf(st.o[k], a, other.o[k] * b);
  st.m = m_new;
}

// Merge the ns partial slots sb .. sb + ns - 1 of rows [r0, r0 + nr) of
// Q-block x and write those output rows (nr * D / 8 <= 256); all 256 threads
// of the workgroup take part.  Thread (group, row, 8 dims): the threads the
// rows do not need form groups that take every groups-th split, and the
// groups' states are merged through `red` (256 entries of LDS), so a Q-block
// cut into many splits (a long decode) is read with many loads in flight;
// each thread issues the loads of four splits before merging them (a split's
// O values are used only when its LSE is finite, so the O loads need not wait
// for the LSE).  ns = 0 writes the empty rows (O = 0,
// LSE = -inf).  COHERENT: the partials were written by other workgroups of
// the running kernel (fused merge).
template <int D, bool OUT_F32, bool COHERENT = false>
__device__ __forceinline__ void merge_rows(const KParams& p, const QBlock& x, int ns, int sb, int r0, int nr,
                                           MergeState* red) {
  const float ninf = -__builtin_huge_valf();
  constexpr int TPR = D / 8;
  const int per = nr * TPR;                          // threads one pass over the rows needs (<= 256)
  const int groups = 256 / per;
  const int t = threadIdx.x;
  const int grp = t / per, idx = t % per;
  const bool live = grp < groups;
  const int row = r0 + idx / TPR, d0 = (idx % TPR) * 8;
  MergeState st;
  st.m = ninf;
  st.z = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = 0.f;
  if (live) {
    const int64_t rs = (int64_t)p.slot_rows;
    for (int sp = grp; sp < ns; sp += 4 * groups) {
      float ls[4];
      f32x4c a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sl = sb + min(sp + u * groups, ns - 1);   // past the last split: re-read it, weight 0 below
        load_part<COHERENT>(p.part_lse + sl * rs + row, p.part_o + (sl * rs + row) * D + d0, ls[u], a[u], b[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (sp + u * groups < ns) merge_part(st, ls[u], a[u], b[u]);
    }
  }
  if (groups > 1) {
    red[t] = st;
    __syncthreads();
    if (live && grp == 0)
      for (int gq = 1; gq < groups; ++gq) merge_state(st, red[gq * per + idx]);
    __syncthreads();
  }
  if (live && grp == 0) {
    const bool empty = !(st.z > 0.f);
    const float inv = empty ? 0.f : 1.f / st.z;
    const float lse = empty ? ninf : st.m + logf(st.z);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = st.o[k] * inv;
    const int tok = x.q0 + x.t0 + row / p.qbh, head = x.g * p.G + row % p.qbh;
    if constexpr (OUT_F32) {
      float* dst = reinterpret_cast<float*>(p.out) + tok * p.o_st + head * p.o_sh + d0;
      *reinterpret_cast<f32x4c*>(dst) = f32x4c{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4c*>(dst + 4) = f32x4c{o[4], o[5], o[6], o[7]};
    } else {
      char* dst = reinterpret_cast<char*>(p.out) + (tok * p.o_st + head * p.o_sh + d0) * 2;
      *reinterpret_cast<u32x4c*>(dst) = u32x4c{pack_bf16x2_c(o[0], o[1]), pack_bf16x2_c(o[2], o[3]),
                                               pack_bf16x2_c(o[4], o[5]), pack_bf16x2_c(o[6], o[7])};
    }
    if (d0 == 0) p.lse[tok * p.l_st + head * p.l_sh] = lse;
  }
}

// Rows per merge chunk: at most eight chunks for the call's largest Q-block
// (slot_rows rows), at least 64 threads' worth of rows; never more than
// 256 / (D / 8) rows for slot_rows <= 128.  The Combine kernel and the fused
// merge cut Q-blocks alike, so they add the splits in the same order.
template <int D>
__device__ __forceinline__ int merge_chunk_rows(const KParams& p) {
  return max(64 / (D / 8), (p.slot_rows + 7) / 8);
}

// Every row of Q-block x, chunk by chunk (one workgroup).
template <int D, bool OUT_F32, bool COHERENT = false>
__device__ __forceinline__ void merge_qblock(const KParams& p, const QBlock& x, int ns, int sb, MergeState* red) {
  const int CR = merge_chunk_rows<D>(p);
  for (int r0 = 0; r0 < x.rows; r0 += CR) {
    merge_rows<D, OUT_F32, COHERENT>(p, x, ns, sb, r0, min(CR, x.rows - r0), red);
    __syncthreads();
  }
}

}  // namespace pa
