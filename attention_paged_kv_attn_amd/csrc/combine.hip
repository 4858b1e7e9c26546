// combine.hip — the Combine stage as a kernel of its own: one workgroup per
// split Q-block merges its partials (the merge itself is in combine_core.h).
#include "combine_core.h"

namespace pa {

// Items are (Q-block, chunk of CR rows), at most eight chunks per Q-block
// (the largest the call can have is slot_rows rows): a chunk of 64 threads
// leaves the workgroup's four thread groups to share its splits, and a wide
// Q-block (a sequence Q-block with every query head) spreads over
// workgroups.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(KParams p) {
  __shared__ MergeState red[256];
  const int CR = merge_chunk_rows<D>(p);
  const int chunks = (p.slot_rows + CR - 1) / CR;
  const bool stat = p.static_S > 0;
  // static split: every Q-block is a candidate, its split count recomputed
  const int n_combine = stat ? p.B * p.Hkv : p.hdr[H_NCOMBINE];
  for (int it = blockIdx.x; it < n_combine * chunks; it += gridDim.x) {
    const int i = it / chunks, r0 = (it - i * chunks) * CR;
    int q, ns, sb;
    QBlock x;
    if (stat) {
      q = i;
      if (static_qblock(p, q, x) != E_NONE) continue;
      ns = static_split(p, x).ns;
      if (ns < 2) continue;                          // written by the attention kernel
      sb = q * p.static_S;
    } else {
      q = p.combine_list[i];
      x = load_qblock(p, q);
      ns = p.n_splits[q];
      sb = p.slot_base[q];
    }
    if (r0 >= x.rows) continue;
    merge_rows<D, OUT_F32>(p, x, ns, sb, r0, min(CR, x.rows - r0), red);
  }
}

hipError_t launch_combine(const KParams& p, bool out_f32, int grid, hipStream_t stream) {
  if (p.D == 64) {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<64, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((combine_kernel<64, false>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((combine_kernel<128, true>), dim3(grid), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((combine_kernel<128, false>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
