// LDS tiles of 64 rows x D bf16 filled by global-to-LDS copies (gfx950).
//
// A tile keeps the source's row-major layout with the 16-byte chunks of
// each row permuted: chunk c of row r sits at slot c ^ swz(r).  The copy
// instruction writes 16 bytes per lane at consecutive LDS addresses, so a
// lane that fills slot s of row r reads source chunk s ^ swz(r).  Three
// permutations, each free of LDS bank conflicts (64 banks of 4 bytes) for
// the reads it serves:
//   k   16-byte operand reads of rows j = 0..15 at one chunk (MFMA operand
//       with the row as the M or N index);
//   v   transposing reads (ds_read_b64_tr_b16) of 4 consecutive rows at 4
//       consecutive chunks, two half-chunks each;
//   kv  both of the above, for a tile read both ways.
#pragma once

#include "common.h"

template <int D> struct TileSwz;
template <> struct TileSwz<128> {  // 16 chunks of 16 B per row
  static __device__ __forceinline__ int k(int r) { return r & 15; }
  static __device__ __forceinline__ int v(int r) { return (r & 3) << 2; }
  static __device__ __forceinline__ int kv(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};
template <> struct TileSwz<64> {   // 8 chunks of 16 B per row
  static __device__ __forceinline__ int k(int r) { return (r >> 1) & 7; }
  static __device__ __forceinline__ int v(int r) { return ((r >> 1) & 1) << 2; }
  static __device__ __forceinline__ int kv(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// 16 bytes per lane from global memory into LDS through a buffer resource
// (MUBUF buffer_load ... lds): lane L of the wave reads 16 bytes at byte
// offset voff of the buffer and writes them at bytes 16 L .. 16 L + 15
// after the wave-uniform address lds.  Unlike the global (FLAT-encoded)
// form, the compiler does not count this copy among the pending
// LDS-counter events, so the operand reads that follow it keep partial
// lgkmcnt waits instead of waiting for every read in flight.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, bf16_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Buffer resource for `bytes` bytes at the wave-uniform address p (gfx9
// descriptor word 3: 32-bit data format, raw addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Wait until this wave's tile copies have landed in LDS (vmcnt(0); the
// copies count on the vector-memory counter only).  A barrier after the
// wait then makes every wave's share of a tile visible to all waves.  The
// immediate is the gfx9 s_waitcnt encoding with vmcnt 0 and the other
// counters at their maximum (expcnt 7, lgkmcnt 15).
__device__ __forceinline__ void tile_copies_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Transposing read: lane 4a+b of each 16-lane group receives element b of
// the 8-byte pieces addressed by lanes a, a+4, a+8 and a+12 of the group.
__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)(__attribute__((address_space(3))) bf16_t*)(p));
}

// A wave's share of a 64-row tile copy: with RPI rows per 1 KB
// instruction and the tile split over NW waves, wave w fills rows
// RPI*(NI*w + q) + lane/CH, q < NI, slot lane%CH of each from source chunk
// slot ^ swz(row); the lane's source byte offsets are worked out once.
// Given a wave-uniform tile address and wave index, each copy instruction
// then addresses memory as scalar descriptor + lane offset and writes LDS
// at a scalar address, so a copy costs no vector arithmetic.
template <int D, int (*SWZ)(int), int NW = 4>  // NW waves share the tile
struct TileCopy {
  static constexpr int CH = D / 8;
  static constexpr int RPI = 1024 / (2 * D);
  static constexpr int NI = 64 / RPI / NW;
  uint32_t off[NI];
  __device__ __forceinline__ void init(int w, int l) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int row = RPI * (NI * w + q) + l / CH, slot = l % CH;
      off[q] = (uint32_t)(row * D + 8 * (slot ^ SWZ(row))) * 2u;
    }
  }
  // src: the tile's first row; w must be wave-uniform.  rows: the rows of
  // the tile that exist in the tensor (64 except for a partial last block);
  // the descriptor covers only those, so no read leaves the tensor.
  __device__ __forceinline__ void copy(const bf16_t* src, bf16_t* dst, int w, int rows = 64) const {
    // the base goes through the scalar unit explicitly (a wave-uniform
    // buffer descriptor)
    const uint64_t a = reinterpret_cast<uint64_t>(src);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), rows * D * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) copy16_to_lds(r, off[q], dst + RPI * (NI * w + q) * D);
  }
};

// Operands of O^T += X^T P^T style products (X = V, K, Q or dO; rows of X
// are the contraction index) from transposing reads: 8 keys 16 s + 4 h +
// {0..3} and 16 s + 8 + 4 h + {0..3} of column 32 dt + lane % 32, built
// from two reads in which lane t of each 16-lane group addresses row
// key0 + t/4, columns 32 dt + 16 (group % 2) + 4 (t % 4) .. +3.  Byte
// offsets of the two reads, split so that k-step s and d tile dt cost one
// XOR-add each: read 1 sits at A1 + ((64 dt) ^ B1) + 32 D s, read 2 at
// A2 + ((64 dt) ^ B2) + 32 D s.  The permutations above depend
// on bits 0-3 of the row only (so k-step s, 16 rows on, moves both reads
// by 32 D bytes), and chunk 4 dt + c0 (c0 < 4) permuted by p is
// 4 (dt ^ (p >> 2)) + (c0 ^ (p & 3)).
template <int D, int (*SWZ)(int)>
__device__ __forceinline__ void col8_parts(int l, uint32_t& A1, uint32_t& B1, uint32_t& A2, uint32_t& B2) {
  const int tg = l & 15, h = l >> 5;
  const int c0 = 2 * ((l >> 4) & 1) + ((tg >> 1) & 1), half = tg & 1;
  const int r1 = 4 * h + (tg >> 2), r2 = r1 + 8;
  const int p1 = SWZ(r1), p2 = SWZ(r2);
  A1 = (uint32_t)(2 * r1 * D + 16 * (c0 ^ (p1 & 3)) + 8 * half);
  A2 = (uint32_t)(2 * r2 * D + 16 * (c0 ^ (p2 & 3)) + 8 * half);
  B1 = (uint32_t)(16 * (p1 & 12));
  B2 = (uint32_t)(16 * (p2 & 12));
}
__device__ __forceinline__ bf16x8 tile_col8_b(const char* t, uint32_t o1, uint32_t o2) {
  return __builtin_shufflevector(ds_read_tr4(reinterpret_cast<const bf16_t*>(t + o1)),
                                 ds_read_tr4(reinterpret_cast<const bf16_t*>(t + o2)), 0, 1, 2, 3, 4, 5, 6, 7);
}
