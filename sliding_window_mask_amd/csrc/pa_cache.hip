// KV-cache write for gfx950: the step before decode. Token t's keys and
// values (all heads) are scattered to physical slot slot_mapping[t] =
// block * 16 + offset of the paged caches [num_blocks, H, 16, D] (the
// block-table layout of "Add Encoder-decoder model support and T5 Model
// support"); a negative slot skips the token (padding).
//
// One workgroup of 256 threads per token: the token's H rows of D elements
// are H * D * e / 16 sixteen-byte pieces; consecutive threads take
// consecutive pieces, so both the read of k_new/v_new and the write into one
// (block, head, slot) row are contiguous 16-byte runs.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWriteThreads = 256;

template <int ROW_BYTES>
__global__ void __launch_bounds__(kWriteThreads) pa_kv_write(KvWriteArgs a) {
  constexpr int kPieces = ROW_BYTES / 16;            // 16-byte pieces per head row
  const int64_t t = blockIdx.x;
  const int64_t slot = a.slot_mapping[t];
  if (slot < 0) return;
  const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
  const int H = a.num_heads;
  const char* ksrc = static_cast<const char*>(a.k_new) + t * H * ROW_BYTES;
  const char* vsrc = static_cast<const char*>(a.v_new) + t * H * ROW_BYTES;
  char* kdst = static_cast<char*>(a.k_cache);
  char* vdst = static_cast<char*>(a.v_cache);
  for (int i = threadIdx.x; i < H * kPieces; i += kWriteThreads) {
    const int h = i / kPieces, c = i % kPieces;
    const int64_t dst = ((blk * H + h) * kBlockSize + off) * ROW_BYTES + c * 16;
    *reinterpret_cast<uint4*>(kdst + dst) =
        *reinterpret_cast<const uint4*>(ksrc + (int64_t)h * ROW_BYTES + c * 16);
    *reinterpret_cast<uint4*>(vdst + dst) =
        *reinterpret_cast<const uint4*>(vsrc + (int64_t)h * ROW_BYTES + c * 16);
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  const int row_bytes = a.head_dim * (a.dtype == 0 ? 4 : 2);
  dim3 grid((unsigned)a.num_tokens);
  switch (row_bytes) {
    case 128: hipLaunchKernelGGL((pa_kv_write<128>), grid, dim3(kWriteThreads), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((pa_kv_write<256>), grid, dim3(kWriteThreads), 0, stream, a); break;
    case 512: hipLaunchKernelGGL((pa_kv_write<512>), grid, dim3(kWriteThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
