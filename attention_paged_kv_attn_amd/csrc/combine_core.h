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

template <bool COHERENT>
__device__ __forceinline__ void merge_part(MergeState& st, float ls, const float* src) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (!(ls > -__builtin_huge_valf())) return;          // an empty part weighs nothing
  f32x4c a, b;
  if constexpr (COHERENT) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = load_coherent(src + k);
      b[k] = load_coherent(src + 4 + k);
    }
  } else {
    a = *reinterpret_cast<const f32x4c*>(src);
    b = *reinterpret_cast<const f32x4c*>(src + 4);
  }
  const float m_new = fmaxf(st.m, ls);
  const float alpha = st.m == -__builtin_huge_valf() ? 0.f : exp2f((st.m - m_new) * kLog2e);
  const float w = exp2f((ls - m_new) * kLog2e);
  st.z = st.z * alpha + w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    st.o[k] = st.o[k] * alpha + w * a[k];
    st.o[4 + k] = st.o[4 + k] * alpha + w * b[k];
  }
  st.m = m_new;
}

__device__ __forceinline__ void merge_state(MergeState& st, const MergeState& other) {
  constexpr float kLog2e = 1.4426950408889634f;
  if (other.m == -__builtin_huge_valf()) return;
  const float m_new = fmaxf(st.m, other.m);
  const float a = st.m == -__builtin_huge_valf() ? 0.f : exp2f((st.m - m_new) * kLog2e);
  const float b = exp2f((other.m - m_new) * kLog2e);
  st.z = st.z * a + other.z * b;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.o[k] = st.o[k] * a + other.o[k] * b;
  st.m = m_new;
}

// Merge the ns partial slots sb .. sb + ns - 1 of Q-block x and write its
// output rows; all 256 threads of the workgroup take part.  Thread (group,
// row, 8 dims): when a Q-block's rows need fewer than 256 threads, the spare
// threads form groups that take every groups-th split, and the groups' states
// are merged through `red` (256 entries of LDS), so that a Q-block cut into
// many splits (a long decode) is read with many loads in flight instead of
// one chain per row.  ns = 0 writes the empty rows (O = 0, LSE = -inf).
// COHERENT: the partials were written by other workgroups of the running
// kernel (fused merge).
template <int D, bool OUT_F32, bool COHERENT = false>
__device__ __forceinline__ void merge_qblock(const KParams& p, const QBlock& x, int ns, int sb, MergeState* red) {
  const float ninf = -__builtin_huge_valf();
  constexpr int TPR = D / 8;
  const int per = x.rows * TPR;                      // threads one pass over the rows needs
  const int groups = per >= 256 ? 1 : 256 / per;
  for (int base = 0; base < per; base += 256) {
    const int t = threadIdx.x;
    const int grp = groups > 1 ? t / per : 0;
    const int idx = groups > 1 ? t % per : base + t;
    const bool live = grp < groups && idx < per;
    const int row = idx / TPR, d0 = (idx % TPR) * 8;
    MergeState st;
    st.m = ninf;
    st.z = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] = 0.f;
    if (live) {
      for (int sp = grp; sp < ns; sp += groups) {
        const float* lp = p.part_lse + (sb + sp) * p.slot_rows + row;
        const float ls = COHERENT ? load_coherent(lp) : *lp;
        merge_part<COHERENT>(st, ls, p.part_o + ((int64_t)(sb + sp) * p.slot_rows + row) * D + d0);
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
      const int tok = x.q0 + x.t0 + row / p.G, head = x.g * p.G + row % p.G;
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
}

}  // namespace pa
