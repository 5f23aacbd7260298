// dQ from stored dS (LongLoRA S2-Attn backward, dQ = scale dS K): the dS tile layout
// shared by the key-major kernel that writes the tiles (attn_bwd.hip) and the kernels that
// read them (dqs_kernel in attn_dsq.hip; hga_dqw_kernel in attn_bwd.hip for the causal local
// part of an HGA segment, one group of S keys), their LDS staging and fragment reads, and
// dqs_kernel's launch.
//
// dS tile layout (64 keys x 64 queries, 8 KB, as the key-major kernel's registers hold it):
// 512 chunks of 16 bytes; chunk ((p * 2 + mq) * 2 + h) * 64 + 32 g + l holds key 32 p + l
// and queries 32 mq + 16 h + 4 g + 0..3 (first 8 bytes) and 32 mq + 16 h + 8 + 4 g + 0..3.
//
// Tiles of one (batch, q head, group) follow each other in lower-triangle order: tile
// (query tile qt, key tile kt <= qt) at qt (qt + 1) / 2 + kt; the (batch, head, group)s at
// ((b H + h) ngroups + grp) times the triangle's tile count.
#pragma once

#include "bwd2_core.h"

namespace s2a {

// dS^T of one 32-query half mq of a 32-key pair, as the key-major kernel holds it (lane
// 32 g + l = key l of the pair, sb[h] = queries 32 mq + 16 h + 4 g + 0..3 then
// 32 mq + 16 h + 8 + 4 g + 0..3): chunks ((mq * 2 + h) * 64 + lane) of the pair's half
// tile, so each store writes 1 KB contiguous.
__device__ __forceinline__ void ds_store_pair(bf16_t* pairbase, const bf16x8_t (&sb)[2], int mq, int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) *reinterpret_cast<bf16x8_t*>(pairbase + ((mq * 2 + h) * 64 + lane) * 8) = sb[h];
}

// In LDS, chunk c of a dS tile (fields p, mq, h, g, l as above) sits at slot s with
// s bits 0-1 = l bits 0-1, bit 2 = g, bit 3 = h,
// bits 4-6 = l bits 2-4, bit 7 = mq, bit 8 = p: the 32 lanes that one transposed read
// serves together then touch 16 distinct 16-byte slots of one 256-byte bank line.
__device__ __forceinline__ int ds_chunk_of_slot(int s) {
  return (s & 0x180) | (((s >> 3) & 1) << 6) | (((s >> 2) & 1) << 5) | (((s >> 4) & 7) << 2) | (s & 3);
}

// LDS element offset of this lane's first transposed read of a dS tile (K-step 0, keys
// 4g .. 4g + 3, query half mq): source lane t of its 16-lane group points at keys
// 4g + t / 4 and queries 32 mq + 16 (lq / 16) + 4 (t % 4) .. + 3.  The second read (keys
// 8 + 4g ..) adds 256 elements, K-step kb adds 512 (kb % 2) + 2048 (kb / 2).
__device__ __forceinline__ int ds_tr_offset(int lane, int mq) {
  const int lq = lane % 32, g = lane / 32, t = lq & 15;
  const int slot = (t >> 2) | ((t & 1) << 2) | ((lq >> 4) << 3) | (g << 4) | (mq << 7);
  return 8 * slot + 4 * ((t >> 1) & 1);
}

__device__ __forceinline__ bf16x8_t ds_frag(const bf16_t* tile, int off, int kb) {
  const bf16_t* a1 = tile + off + 512 * (kb & 1) + 2048 * (kb >> 1);
  const s16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)a1);
  const s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)(a1 + 256));
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  return as_bf16x8(uint4{ux.x, ux.y, uy.x, uy.y});
}

// One 16-byte piece per lane of a dS tile copied into LDS (64 lanes fill 1 KB from
// lds_wave_base).  The tiles are read once: the copies carry the non-temporal hint (cache
// policy nt), so they do not push the K tiles, which every unit of a group re-reads, out of
// the L2 (158 -> 144 us for the dQ kernel at N=8192, H=32).
__device__ __forceinline__ void load_lds16_stream(const bf16_t* src, bf16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 2);
}

// dQ (bf16, token order, [B, N, H, d]) = scale dS K for every (batch, head, group), from
// the tiles at dsw; d = 64 or 128.  Launches one kernel on st.
void launch_dqs(int d, const bf16_t* k, const bf16_t* dsw, bf16_t* dq, int B, int N, int H, int Hkv, int G,
                int shift, float scale, hipStream_t st);

}  // namespace s2a
