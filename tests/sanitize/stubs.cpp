// Stand-ins for the device-side units of the library, so that the host code
// (tri_attn.cpp) can be built on its own with the address and
// undefined-behaviour sanitizers and its argument paths run on a machine
// without a GPU. Every launch fails; nothing here is reached by those paths
// except `supported`, which keeps the library's rule.
#include "tri_attn.h"
#include "tri_attn_internal.h"

namespace tpa {
bool supported(int D, int dh) { return (D == 64 || D == 128) && (dh == 16 || dh == 32); }
int k2_items(int, int, int, int B, int N) { return B * N; }
int k1_blocks_per_cu(int, int, int) { return 1; }
int k2_blocks_per_cu(int, int, int) { return 1; }
int k3_blocks_per_cu(int, int) { return 1; }
int k1_split_blocks_per_cu(int, int) { return 1; }
size_t bwd_workspace_bytes(int B, int N, int D, int h, int, int, int) { return (size_t)B * N * N * (5 * D + h) * 16; }
int scratch_address(int, void **ptr) {
  *ptr = nullptr;
  return TRI_ATTN_ERR_HIP;
}
hipError_t launch_k1(int, int, int, const K1Args &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_k1_split(int, int, const K1Args &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_k2(int, int, int, const K2Args &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_k3(int, int, const K3Args &, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_k2_train(int, int, const K2Args &, const K2TrainArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_bwd(int, int, int, const BwdRunArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_onepass(int, int, int, const OnePassArgs &, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_pack_frags(int, int, const void *, void *, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_pack_frags_split3(int, const void *, void *, size_t, int, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace tpa
