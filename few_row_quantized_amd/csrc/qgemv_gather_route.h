// Routing of a gathered (MoE) verify, resolved on the device by every
// workgroup that needs it (the routing never goes to the host).  Shared by
// the single-pass MFMA kernel's gathered variant (qgemv_mfma_impl.h) and the
// persistent one (qgemv_persist.hip).
#pragma once

#include "qgemv_device.h"
#include "qgemv_internal.h"

namespace qgemv {

// Reads the P pairs into LDS and orders the valid ones (expert in [0, E),
// activation row in [0, X)) by (expert, pair) with a stable rank sort (the
// position of a valid pair counts the valid pairs with a smaller expert, or
// the same expert and a smaller index); the runs of equal experts become the
// slots, in ascending expert order.  All threads of the workgroup call it;
// on return (after a workgroup barrier):
//   gexp[p]       expert of pair p, -1 if the pair is invalid
//   gxr[p]        activation row of pair p
//   gsorted[i]    the i-th valid pair in (expert, pair) order, i < nvalid
//   gstart[s]     first position of slot s; gstart[nslots] = nvalid
//   gslot_exp[s]  expert of slot s
//   gmeta[0]      nslots
// Arrays of kMaxPairs entries (gstart: kMaxPairs + 1); P <= kMaxPairs.
__device__ __forceinline__ void gather_route(const GatherArgs &ga, int *gexp, int *gxr, int *gsorted,
                                             int *gstart, int *gslot_exp, int *gmeta) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int p = threadIdx.x; p < ga.P; p += blockDim.x) {
    const int e = ga.e_idx[p], xi = ga.x_idx[p];
    const bool valid = e >= 0 && e < ga.E && xi >= 0 && xi < ga.X;
    gexp[p] = valid ? e : -1;
    gxr[p] = xi;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < ga.P; p += blockDim.x) {
    const int e = gexp[p];
    if (e < 0) continue;
    int rank = 0;
    for (int q = 0; q < ga.P; ++q) {
      const int f = gexp[q];
      rank += (f >= 0 && (f < e || (f == e && q < p))) ? 1 : 0;
    }
    gsorted[rank] = p;
  }
  int nvalid = 0;
  if (wave == 0) {
    for (int p0 = 0; p0 < ga.P; p0 += 64) {
      const int p = p0 + lane;
      nvalid += __popcll(__ballot(p < ga.P && gexp[p] >= 0));
    }
  }
  __syncthreads();
  if (wave == 0) {
    // slot boundaries: a position whose expert differs from the one before
    int base = 0;
    for (int i0 = 0; i0 < nvalid; i0 += 64) {
      const int i = i0 + lane;
      int e = -1;
      bool first = false;
      if (i < nvalid) {
        e = gexp[gsorted[i]];
        first = i == 0 || gexp[gsorted[i - 1]] != e;
      }
      const uint64_t bal = __ballot(first);
      if (first) {
        const int sl = base + __popcll(bal & ((1ull << lane) - 1ull));
        gstart[sl] = i;
        gslot_exp[sl] = e;
      }
      base += __popcll(bal);
    }
    if (lane == 0) {
      gmeta[0] = base;
      gstart[base] = nvalid;
    }
  }
  __syncthreads();
}

}  // namespace qgemv
