// MXFP4 scale packing: E8M0 scale bytes [E, N, K/32] (row n, MX block kb) -> records of
// kMxRecRows rows x kMxRecBlocks bytes, one per (expert, 64-row block of N, 8 MX blocks
// of K), the order in which the grouped GEMMs read them.  A wave of the decode tiling then
// fetches the scales of a record's 64 B-rows for a 256-element K range with one 8-byte
// load per lane (512 contiguous bytes) instead of one line per B-row.
#include "moe_launch.h"

namespace moe {
namespace {

// Thread i writes the 8 bytes of record row i = ((e * NB + nb) * KR + kr) * 64 + r:
// MX blocks 8 kr .. 8 kr + 7 of row 64 nb + r of expert e; blocks past K/32 are zero.
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst,
                                                             int64_t nruns, int KB, int KR) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= nruns) return;
  const int r = static_cast<int>(i % kMxRecRows);
  const int64_t rec = i / kMxRecRows;                    // (e * NB + nb) * KR + kr
  const int kr = static_cast<int>(rec % KR);
  const int64_t row = (rec / KR) * kMxRecRows + r;       // e * N + 64 nb + r
  const uint8_t* s = src + row * KB;
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < kMxRecBlocks; ++j) {
    const int kb = kMxRecBlocks * kr + j;
    const uint32_t v = kb < KB ? s[kb] : 0u;
    w[j >> 2] |= v << (8 * (j & 3));
  }
  reinterpret_cast<uint2*>(dst)[i] = make_uint2(w[0], w[1]);
}

}  // namespace

hipError_t launch_pack_mx_scales(const uint8_t* src, uint8_t* dst, int64_t E, int64_t N,
                                 int64_t K, hipStream_t stream) {
  const int64_t KR = mx_rec_k(K);
  const int64_t nruns = E * (N / kMxRecRows) * KR * kMxRecRows;
  if (nruns == 0) return hipSuccess;
  const int64_t blocks = (nruns + 255) / 256;
  hipLaunchKernelGGL(pack_mx_scales_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, src, dst, nruns, static_cast<int>(K / 32), static_cast<int>(KR));
  return hipGetLastError();
}

}  // namespace moe
