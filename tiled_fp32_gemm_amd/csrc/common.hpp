// common.hpp -- device helpers shared by the gfx950 SGEMM kernels.
//
// Buffer resources.  Every operand is read and written through a raw buffer
// resource (base, byte size).  A kernel does not address a whole operand from
// its first element: it moves the base to the corner of its own C tile (A to
// the tile's first row, C to its first row and column, B to its first column
// and, slab by slab, to the slab's first row), so that every byte offset a
// lane forms stays below 2^31 however large the operand is; the host checks
// that one tile's rows of A (over all of K) and of C, and one slab's rows of
// B, span less than 2 GiB.  A
// resource is never larger than 2^31 bytes, and a lane whose element lies
// outside the logical matrix is given the byte offset kOob = 2^31, past its
// end, so its load returns 0 and its store is dropped by the hardware range
// check.  That is the pages' predicated edge load that writes 0 for invalid
// elements ("CUDA in depth (5)", section on edges), without a branch, and no
// stale value is ever multiplied by 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a gfx9-family buffer descriptor: 32-bit data format, raw (no
// swizzle, stride 0) addressing.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOob = 0x80000000u;
constexpr int64_t kRsrcMax = int64_t(1) << 31;  // bytes; kOob is past the end

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ f32x4 load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                       float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off,
                                        0, 0);
}

// store1 with the nontemporal hint (cache-policy bit 1, "nt" on gfx950): for
// a product's C, which is written once and not read back by the kernel.
// Measured on MI355X against plain stores, same bits: +6% at 65536 x 128 x
// 256, whose 32 MiB C store is a seventh of the launch, and level to +1% on
// square and ragged shapes.  Not for split partials, which the reduction
// reads straight back.
__device__ __forceinline__ void store1_nt(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                          float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off,
                                        0, 2);
}

// Two adjacent words, plain or with the nontemporal hint.
__device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                       f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}

__device__ __forceinline__ void store2_nt(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                          f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 2);
}

__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                       f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off,
                                         0, 0);
}

// min(rem, cap) for a wave-uniform rem >= 0 and cap <= 2^31, formed with
// 32-bit scalar operations on the two halves: the scalar unit has no 64-bit
// ordered compare, and a 64-bit one would move the clamp to the vector unit
// and put a branch in the slab loop.  The empty asm keeps the compiler from
// folding the halves back into one 64-bit compare.
__device__ __forceinline__ uint32_t cap_bytes(uint64_t rem, uint32_t cap) {
  uint32_t hi = (uint32_t)(rem >> 32), lo = (uint32_t)rem;
  asm volatile("" : "+s"(hi), "+s"(lo));
  const uint32_t m = lo < cap ? lo : cap;
  return hi != 0u ? cap : m;
}

// A resource over an operand of `bytes` bytes starting at `base`, moved
// `skip` floats forward (skip * 4 < bytes): the rest of the operand, capped
// at kRsrcMax bytes.  All arguments are wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const float* base,
                                                        int64_t bytes,
                                                        int64_t skip) {
  return make_rsrc(base + skip, cap_bytes((uint64_t)(bytes - 4 * skip), (uint32_t)kRsrcMax));
}

// The resource of the K slab starting at column k0 of a tile's rows of A:
// from base + k0 (base: the tile's first row), cap - 4 k0 bytes, where cap is
// the capped size of the whole rest of A from base (rsrc_at's size with
// skip 0).  Exact, and 32-bit only, because the host checks that a tile's
// rows of A over all of K span less than 2^31 bytes: words below K lie
// inside it whether or not cap was capped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_slab_a(const float* base,
                                                            uint32_t cap, int k0) {
  return make_rsrc(base + k0, cap - 4u * (uint32_t)k0);
}

// 16 bytes per lane from global memory straight into LDS: lane l's data lands
// at lds_dst + 16 l bytes (lds_dst must be the same for the whole wave);
// out-of-range lanes write zeros.
__device__ __forceinline__ void load4_to_lds(__amdgpu_buffer_rsrc_t r,
                                             float* lds_dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_dst, 16, off, 0, 0, 0);
}

// Kernel arguments, identical for every family.  Sizes are checked on the
// host: 0 <= M, N, K < 2^31 - 1024 (so tile origins stay in int range) and one
// tile's rows of A and C, and one slab's rows of B, span less than 2 GiB, so
// 32-bit byte offsets from a tile's corner suffice.
struct GemmArgs {
  const float* A;
  const float* B;
  float* C;
  int64_t a_bytes, b_bytes, c_bytes;   // bytes each operand spans
  int M, N, K;
  int lda, ldb, ldc;
  int tiles_m, tiles_n;                // C tiles along M and N
  int group_m;                         // tile rows per ordering group
  // Split K across workgroups (kernels instantiated for it only): split s
  // covers k in [s k_split, min((s + 1) k_split, K)) and writes its partial
  // tile to W + s M N (rows of N floats).
  int splits, k_split;
  float* W;
};

// Workgroup -> C tile.  Workgroups are handed to the 8 XCDs round-robin
// (workgroup w runs on XCD w % 8), and each XCD has its own L2.  The id is
// first renumbered so that ids running on one XCD are consecutive, then
// consecutive ids walk a group of group_m tile rows column by column, so the
// tiles one XCD holds at a time share A row panels and B column panels.
__device__ __forceinline__ void tile_of_workgroup(const GemmArgs& g, int& tm,
                                                  int& tn) {
  const int nwg = g.tiles_m * g.tiles_n;
  const int w = (int)blockIdx.x;
  const int q = nwg >> 3, rem = nwg & 7;
  const int xcd = w & 7, local = w >> 3;
  const int L = xcd * q + (xcd < rem ? xcd : rem) + local;
  const int per_group = g.group_m * g.tiles_n;
  const int grp = L / per_group;
  const int first_m = grp * g.group_m;
  const int rows = min(g.tiles_m - first_m, g.group_m);
  const int in_grp = L - grp * per_group;
  tm = first_m + in_grp % rows;
  tn = in_grp / rows;
}

// Workgroup -> (split, C tile) for a grid of splits x tiles workgroups: the
// same XCD renumbering over the whole grid, split-major, so that an XCD holds
// neighbouring tiles of one K range at a time.
__device__ __forceinline__ void tile_split_of_workgroup(const GemmArgs& g, int& tm,
                                                        int& tn, int& split) {
  const int tiles = g.tiles_m * g.tiles_n;
  const int nwg = tiles * g.splits;
  const int w = (int)blockIdx.x;
  const int q = nwg >> 3, rem = nwg & 7;
  const int xcd = w & 7, local = w >> 3;
  int L = xcd * q + (xcd < rem ? xcd : rem) + local;
  split = L / tiles;
  L -= split * tiles;
  const int per_group = g.group_m * g.tiles_n;
  const int grp = L / per_group;
  const int first_m = grp * g.group_m;
  const int rows = min(g.tiles_m - first_m, g.group_m);
  const int in_grp = L - grp * per_group;
  tm = first_m + in_grp % rows;
  tn = in_grp / rows;
}

}  // namespace sg
