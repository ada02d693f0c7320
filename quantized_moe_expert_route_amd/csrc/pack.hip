// One-time rewrite of the routed experts' gate/up weights into the layout
// the gate/up kernels stream: expert weights are repacked for the kernel
// once, when they are loaded ("IQ2R: load GLM-5.3 packed MoE checkpoints
// with TP slicing", Summary: the MoE method allocates packed expert tensors
// at load time; "[HIP] IQ2R: GLM-5.3 packed MoE path for TP4/TP8 on
// gfx950", file list: packing into the kernel's layout is part of the path).
//
// Row-major MXFP4 gate/up weights [E, 2I, H/2] put one 16-row, 64-byte piece
// of a K-step (128 elements) into 16 separate cache lines, so a load whose
// lanes cover it costs the memory pipeline about four times one that covers
// 1 KB contiguous bytes. Packed, that piece is 1 KB contiguous and in the
// scaled FP4 MFMA's operand order (lane 16 g + r holds row r, bytes 16 g ..
// 16 g + 15 of the K-step: MX block g), so lane l's 16 bytes are bytes
// 16 l .. 16 l + 15 of the piece:
//   w13p [E * 2I/16 row blocks][H/128 K-steps][4 groups g][16 rows r][16 bytes]
// and the E8M0 scales of a row block's 512-wide stage are 256 contiguous
// bytes, ordered the same way (lane group g, then row r, then the four
// K-steps j of the stage):
//   s13p [E * 2I/16][H/512 stages][4 groups g][16 rows r][4 steps j]
// holding the scale of MX block 16 * stage + 4 j + g of row 16 * block + r.
// Both are byte permutations of the inputs: nothing is rounded.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

__global__ __launch_bounds__(256) void pack_w13_kernel(const uint8_t* __restrict__ w, uint8_t* __restrict__ wp,
                                                       int64_t units, int nks, int64_t row_bytes) {
  // unit o: bytes 16 g .. of row r of (row block rb, K-step ks)
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < units; o += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(o & 15), g = (int)((o >> 4) & 3);
    const int64_t rest = o >> 6;
    const int ks = (int)(rest % nks);
    const int64_t rb = rest / nks;
    *reinterpret_cast<uint4*>(wp + 16 * o) =
        *reinterpret_cast<const uint4*>(w + (rb * 16 + r) * row_bytes + 64 * ks + 16 * g);
  }
}

__global__ __launch_bounds__(256) void pack_s13_kernel(const uint8_t* __restrict__ s, uint32_t* __restrict__ sp,
                                                       int64_t dwords, int nkq, int64_t row_bytes) {
  // dword d: the four K-steps of lane (g, r) of (row block rb, stage kq)
  for (int64_t d = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; d < dwords; d += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(d & 15), g = (int)((d >> 4) & 3);
    const int64_t rest = d >> 6;
    const int kq = (int)(rest % nkq);
    const int64_t rb = rest / nkq;
    const uint8_t* src = s + (rb * 16 + r) * row_bytes + 16 * kq + g;
    sp[d] = (uint32_t)src[0] | ((uint32_t)src[4] << 8) | ((uint32_t)src[8] << 16) | ((uint32_t)src[12] << 24);
  }
}

// Down weights for the MXFP4-mid down (rows are output columns, K = I <= 512,
// so at most four K-steps): dword d of row block rb holds, for lane (g, r),
// the scale bytes of MX blocks 4 ks + g of row 16 rb + r in byte ks, ks <
// nks; the other bytes are zero.
__global__ __launch_bounds__(256) void pack_s2_kernel(const uint8_t* __restrict__ s, uint32_t* __restrict__ sp,
                                                      int64_t dwords, int nks, int64_t row_bytes) {
  for (int64_t d = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; d < dwords; d += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(d & 15), g = (int)((d >> 4) & 3);
    const int64_t rb = d >> 6;
    const uint8_t* src = s + (rb * 16 + r) * row_bytes + g;
    uint32_t v = 0;
    for (int ks = 0; ks < nks; ++ks) v |= (uint32_t)src[4 * ks] << (8 * ks);
    sp[d] = v;
  }
}

hipError_t launch_pack_w2(const void* w2, const void* s2, int64_t E, int64_t I, int64_t H, void* w2p, void* s2p,
                          hipStream_t stream) {
  const int64_t rows = E * H;
  const int64_t units = rows * (I / 32);  // 16-byte units of w2
  const int64_t dwords = rows * 4;        // one dword per lane per 16-row block
  auto blocks = [](int64_t n) { return (int)std::min<int64_t>((n + 255) / 256, 65536); };
  hipLaunchKernelGGL(pack_w13_kernel, dim3(blocks(units)), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(w2), reinterpret_cast<uint8_t*>(w2p), units, (int)(I / 128),
                     I / 2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_s2_kernel, dim3(blocks(dwords)), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(s2), reinterpret_cast<uint32_t*>(s2p), dwords, (int)(I / 128),
                     I / 32);
  return hipGetLastError();
}

hipError_t launch_pack_w13(const void* w13, const void* s13, int64_t E, int64_t I, int64_t H, void* w13p, void* s13p,
                           hipStream_t stream) {
  const int64_t rows = E * 2 * I;
  const int64_t units = rows * (H / 32);   // 16-byte units of w13
  const int64_t dwords = rows * (H / 128); // dwords of s13
  auto blocks = [](int64_t n) { return (int)std::min<int64_t>((n + 255) / 256, 65536); };
  hipLaunchKernelGGL(pack_w13_kernel, dim3(blocks(units)), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(w13), reinterpret_cast<uint8_t*>(w13p), units, (int)(H / 128),
                     H / 2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pack_s13_kernel, dim3(blocks(dwords)), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(s13), reinterpret_cast<uint32_t*>(s13p), dwords, (int)(H / 512),
                     H / 32);
  return hipGetLastError();
}

}  // namespace qmoe
