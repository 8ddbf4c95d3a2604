// Device-side padding mask from cu_seqlens (TransformerEngine PR #24, "Build
// the attention padding mask without host syncs", Description and Changes):
// mask[b, p] = p >= cu[b+1] - cu[b] for b < B, p < max_seqlen; entries past
// cu[B] are never read. One byte per position (torch.bool layout); each
// thread builds 16 consecutive bytes of the flattened [B, max_seqlen] mask and
// writes them with one 16-byte store (byte stores when the buffer is not
// 16-byte aligned or at the ragged end).
#include "device.hpp"
#include "launch.hpp"

namespace vattn {

__device__ __forceinline__ int len_i32(const int32_t* cu, int64_t b) {
  return (int)((uint32_t)cu[b + 1] - (uint32_t)cu[b]);  // int32 wraparound
}

// Grid-stride body shared by the single and the cross-attention kernels.
__device__ __forceinline__ void build_mask(const int32_t* __restrict__ cu, int max_seqlen,
                                           int64_t total, uint8_t* __restrict__ mask, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 16;
  for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; base < total;
       base += stride) {
    int64_t b = base / max_seqlen;
    int p = (int)(base - b * max_seqlen);
    int len = len_i32(cu, b);
    uint32_t wd[4] = {0, 0, 0, 0};
    const int n = (total - base) < 16 ? (int)(total - base) : 16;
    for (int j = 0; j < n; ++j) {
      if (p >= len) wd[j >> 2] |= 1u << ((j & 3) * 8);
      if (++p == max_seqlen && j + 1 < n) {
        p = 0;
        ++b;
        len = len_i32(cu, b);
      }
    }
    if (vec && n == 16) {
      st16(mask + base, u32x4{wd[0], wd[1], wd[2], wd[3]});
    } else {
      for (int j = 0; j < n; ++j) mask[base + j] = (uint8_t)((wd[j >> 2] >> ((j & 3) * 8)) & 1u);
    }
  }
}

__global__ __launch_bounds__(256) void padding_mask_kernel(const int32_t* __restrict__ cu,
                                                           int max_seqlen, int64_t total,
                                                           uint8_t* __restrict__ mask,
                                                           int vec) {
  build_mask(cu, max_seqlen, total, mask, vec);
}

// Cross attention (TransformerEngine PR #24, Equivalence: query-side and
// key-side masks of one batch): blockIdx.y = 0 builds the query mask, 1 the
// key mask, in one launch.
struct MaskSide {
  const int32_t* cu;
  uint8_t* mask;
  int64_t total;
  int max_seqlen;
  int vec;
};

__global__ __launch_bounds__(256) void cross_padding_mask_kernel(MaskSide q, MaskSide kv) {
  const MaskSide& m = blockIdx.y == 0 ? q : kv;
  if (m.total == 0) return;
  build_mask(m.cu, m.max_seqlen, m.total, m.mask, m.vec);
}

__global__ void clear_word_kernel(int32_t* w) {
  if (threadIdx.x == 0) *w = 0;
}

hipError_t launch_padding_mask(const int32_t* cu, int B, int max_seqlen, uint8_t* mask,
                               hipStream_t st) {
  const int64_t total = (int64_t)B * max_seqlen;
  if (total == 0) return hipSuccess;
  const int64_t chunks = (total + 15) / 16;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const int vec = ((uintptr_t)mask & 15) == 0;
  padding_mask_kernel<<<(unsigned)blocks, 256, 0, st>>>(cu, max_seqlen, total, mask, vec);
  return hipGetLastError();
}

static int64_t mask_blocks(int64_t total) {
  const int64_t chunks = (total + 15) / 16;
  const int64_t blocks = (chunks + 255) / 256;
  return blocks > 65536 ? 65536 : blocks;
}

hipError_t launch_cross_padding_mask(const int32_t* cu_q, const int32_t* cu_kv, int B,
                                     int max_q, int max_kv, uint8_t* mask_q, uint8_t* mask_kv,
                                     hipStream_t st) {
  MaskSide q{cu_q, mask_q, (int64_t)B * max_q, max_q, ((uintptr_t)mask_q & 15) == 0};
  MaskSide kv{cu_kv, mask_kv, (int64_t)B * max_kv, max_kv, ((uintptr_t)mask_kv & 15) == 0};
  const int64_t blocks = mask_blocks(q.total > kv.total ? q.total : kv.total);
  if (blocks == 0) return hipSuccess;
  cross_padding_mask_kernel<<<dim3((unsigned)blocks, 2), 256, 0, st>>>(q, kv);
  return hipGetLastError();
}

hipError_t launch_clear_word(int32_t* word, hipStream_t st) {
  clear_word_kernel<<<1, 64, 0, st>>>(word);
  return hipGetLastError();
}

}  // namespace vattn
