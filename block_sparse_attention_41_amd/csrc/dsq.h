// dQ from stored dS (LongLoRA S2-Attn backward, dQ = scale dS K): the dS tile layout
// shared by the key-major kernel that writes the tiles (attn_bwd.hip) and dqs_kernel that
// reads them (attn_dsq.hip), and that kernel's launch.
//
// dS tile layout (64 keys x 64 queries, 8 KB, as the key-major kernel's registers hold it):
// 512 chunks of 16 bytes; chunk ((p * 2 + mq) * 2 + h) * 64 + 32 g + l holds key 32 p + l
// and queries 32 mq + 16 h + 4 g + 0..3 (first 8 bytes) and 32 mq + 16 h + 8 + 4 g + 0..3.
//
// Tiles of one (batch, q head, group) follow each other in lower-triangle order: tile
// (query tile qt, key tile kt <= qt) at qt (qt + 1) / 2 + kt; the (batch, head, group)s at
// ((b H + h) ngroups + grp) times the triangle's tile count.
#pragma once

#include "common.h"

namespace s2a {

// dS^T of one 32-query half mq of a 32-key pair, as the key-major kernel holds it (lane
// 32 g + l = key l of the pair, sb[h] = queries 32 mq + 16 h + 4 g + 0..3 then
// 32 mq + 16 h + 8 + 4 g + 0..3): chunks ((mq * 2 + h) * 64 + lane) of the pair's half
// tile, so each store writes 1 KB contiguous.
__device__ __forceinline__ void ds_store_pair(bf16_t* pairbase, const bf16x8_t (&sb)[2], int mq, int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) *reinterpret_cast<bf16x8_t*>(pairbase + ((mq * 2 + h) * 64 + lane) * 8) = sb[h];
}

// dQ (bf16, token order, [B, N, H, d]) = scale dS K for every (batch, head, group), from
// the tiles at dsw; d = 64 or 128.  Launches one kernel on st.
void launch_dqs(int d, const bf16_t* k, const bf16_t* dsw, bf16_t* dq, int B, int N, int H, int Hkv, int G,
                int shift, float scale, hipStream_t st);

}  // namespace s2a
