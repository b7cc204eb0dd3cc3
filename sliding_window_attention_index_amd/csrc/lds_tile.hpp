// LDS tiles of 32 bf16 rows filled by direct global->LDS DMA
// (buffer_load_dwordx4 ... lds, gfx950), shared by the MFMA kernels.
//
// A tile holds 32 rows of D bf16 (D in {64, 128}) without padding.  Inside a
// row, 16-byte chunk c is stored at physical chunk c ^ swz(row).  The
// swizzle makes both LDS access patterns of the attention kernels
// bank-conflict free:
//   * 16-byte reads of one logical chunk by 16 consecutive rows (the
//     A operand of S^T = K . Q^T), and
//   * ds_read_b64_tr_b16 of 4 consecutive rows x 16 dims (the V^T operand of
//     O^T = V^T . P^T).
// One DMA instruction writes 64 lanes x 16 bytes = 1 KiB of consecutive LDS,
// so the swizzle is applied by choosing which global chunk each lane fetches.
#pragma once

#include "sattn_device.hpp"

namespace sattn {

typedef __attribute__((address_space(3))) void lds_void_t;

template <int D>
struct SwizzledTile {
  static constexpr int kRows = 32;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  static constexpr int kBytes = kRows * kRowBytes;
  static constexpr int kDmaPerTile = kBytes / 1024;  // wave-wide DMA instructions per tile

  // Physical chunk of logical chunk c in row r: c ^ f(r).  The LDS serves 256 bytes (64 banks of
  // 4 bytes) a clock: a 16-byte read of 64 lanes goes 16 lanes at a time, an 8-byte read 32 lanes at
  // a time.  f is chosen so that both of these are conflict free:
  //   * 16 consecutive rows (16k .. 16k + 15) reading one logical chunk (the K operand): f takes
  //     distinct values on the rows of the group that share a 256-byte bank window position;
  //   * 4 consecutive rows (4k .. 4k + 3) reading an aligned run of 4 chunks with
  //     ds_read_b64_tr_b16 (the V^T operand, 32 lanes = 4 rows x 4 chunks x 8 bytes): the rows
  //     that share bank positions differ in bit 2 of f, so their chunk runs do not overlap.
  // D = 128 (256-byte rows): f(r) = 4 (r % 4) + (r / 4) % 4.  D = 64 (128-byte rows, two to a bank
  // window, even and odd rows on opposite halves): f(r) = 4 ((r / 2) % 2) + (r / 4) % 4.
  __device__ static __forceinline__ int phys(int r, int c) {
    if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // f(r + 8) = f(r) ^ 2 and f(r + 16) = f(r): a read 8 rows further (an immediate offset of
  // 8 rows) finds logical chunk c at the address of chunk c ^ 2 of its own row, i.e. the byte
  // address XORed with kRow8Xor; 16 rows further, at the same address.
  static constexpr uint32_t kRow8Xor = 32;
  // Byte offset inside the tile of logical chunk c of row r.
  __device__ static __forceinline__ int offset(int r, int c) { return r * kRowBytes + phys(r, c) * 16; }

  // For DMA instruction `slot` (0..kDmaPerTile-1) and lane l: the tile row and
  // the logical chunk this lane must fetch.
  __device__ static __forceinline__ void dma_source(int slot, int l, int &row, int &chunk) {
    const int p = slot * 1024 + l * 16;
    row = p / kRowBytes;
    chunk = phys(row, (p % kRowBytes) / 16);  // the swizzle is an involution
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// One 16-byte DMA per lane from rsrc + voffset into lds (+16 * lane).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, void *lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds), 16, voffset, 0, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (vmcnt only: expcnt and lgkmcnt are left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ bf16x4 lds_read_tr(const void *p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)(p)));
}

// LDS reads the compiler does not see.  Reads of a ring slot that DMA fills
// would otherwise make the compiler wait for every outstanding DMA (vmcnt(0));
// here the caller owns both counters: vmcnt through wait_vmcnt before the
// barrier that publishes a slot, lgkmcnt through lgkm_fence, which also ties
// the loaded registers so that nothing consumes them before the wait.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read_b128(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr_b16(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// LDS write the compiler does not see (for wave-private staging next to DMA buffers).  A wave's
// LDS instructions execute in order, so a later ds_read of the same bytes by this wave sees it.
template <int OFF>
__device__ __forceinline__ void ds_write_b128(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_write_b64(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(addr), "v"(v), "i"(OFF));
}
// A buffer store of more than 64 bits reads its data registers after it issues, and a VALU write
// of those registers right behind it changes what is stored; the compiler pads this case only when
// the store's offset is not an SGPR.  Stores with an SGPR offset go through here: the data stays
// live, and therefore unwritten, until two wait states after the store.
__device__ __forceinline__ void buffer_store_b128_sgpr(u32x4 v, __amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                                       uint32_t soffset) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, voffset, soffset, 0);
  asm volatile("s_nop 1" ::"v"(v));
}

// s_waitcnt lgkmcnt(N) that the registers in `regs` depend on.
template <int N, typename T, int M>
__device__ __forceinline__ void lgkm_fence(T (&regs)[M]) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N));
#pragma unroll
  for (int i = 0; i < M; ++i) asm volatile("" : "+v"(regs[i]));
}

}  // namespace sattn
