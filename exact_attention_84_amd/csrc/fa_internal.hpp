// Host <-> kernel interface of the attention library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fa_fastdiv.hpp"

namespace fa {

// Prefill tile shape of the 32-row kernels (head dim 64, the score variants,
// FP8): 4 waves per workgroup, each owning kFwdNT groups of 32 query rows;
// K/V tiles of 64 keys.  The 64-row kernel takes 2 or 4 waves of 64 rows.
#ifndef FA_FWD_NT
#define FA_FWD_NT 1
#endif
constexpr int kFwdNT = FA_FWD_NT;

// Split-KV decode: a workgroup of 4 waves takes 128 keys per step, 32 per wave.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeTile = 128;
constexpr int kDecodeMaxGroup = 32;
constexpr int kCombineMaxSplits = 4096;
constexpr float kLog2eHost = 1.4426950408889634f;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  const int32_t* cu_q;  // NULL: fixed-length batch
  const int32_t* cu_k;
  int hq, hkv, group;
  int seqlen_q, seqlen_k;  // fixed-length mode
  int n_qtiles;            // query tiles per (sequence, head), longest sequence
  int n_items;             // workgroups per (sequence, head): n_qtiles, or
                           // ceil(n_qtiles / 2) when causal tiles are paired
  int total;               // workgroups
  int waves;               // waves per workgroup
  int wide;                // 1: the 64-row-wave kernel (head dim 128), 0: 32-row waves
  float c;                 // scale * log2(e); 1 where scores arrive in log2 units
  int o_f32;
  // work-item decode of the 64-row kernel by division with precomputed
  // multipliers: items per (sequence, head), query heads per kv head, kv
  // heads, and the XCD deal's group size (group * n_items) with the first
  // block index past its complete rounds of 8 groups
  FastDiv fd_items, fd_group, fd_hkv, fd_gs;
  int remap_end;
};

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cache_seqlens;
  float* o_part;    // [B*Hq][n_splits][D]
  float* lse_part;  // [B*Hq][n_splits]
  int hq, hkv, group;
  int cache_len;    // rows per sequence (capacity)
  int chunk;
  int n_splits;
  int total;  // B * Hkv * n_splits
  float c;
  // paged cache (block_table != nullptr): [num_blocks][page_size][Hkv][D],
  // logical row j of sequence b in block block_table[b * max_blocks + j / page_size]
  const int32_t* block_table;
  int max_blocks, page_size, num_blocks;
  int len_add;  // keys attended = cache_seqlens[b] + len_add (1 after an append)
};

// In-place append of one new token per sequence with rotary embedding.
struct AppendParams {
  const uint16_t* q;      // [B][Hq][D]
  const uint16_t* k_new;  // [B][Hkv][D] or nullptr
  const uint16_t* v_new;
  uint16_t* q_rot;        // [B][Hq][D] or nullptr (no rotary)
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* cache_seqlens;
  const int32_t* block_table;
  int max_blocks, page_size, num_blocks;
  const float* cos;       // [max_pos][rdim / 2] or nullptr
  const float* sin;
  int rdim, max_pos, interleaved;
  int batch, hq, hkv, cache_len;
};

// Backward.  The workspace holds two fp32 arrays [Hq][rows_cap + pad]:
// D = rowsum(dO * O) and LSE * log2(e), head-major so that a lane can read
// four consecutive query rows at once.
constexpr int kBwdPad = 64;  // rows of padding after each head's rows

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;       // [rows, Hq], natural log
  float* dsum;            // workspace: D [Hq][rows_cap + kBwdPad]
  float* lse2;            // workspace: LSE * log2(e), same layout
  void* dq;               // [rows, Hq, d]
  void* dk;               // [key rows, Hkv, d]
  void* dv;
  const int32_t* cu_q;    // NULL: fixed-length batch
  const int32_t* cu_k;
  int batch, hq, hkv, group;
  int seqlen_q, seqlen_k;  // fixed-length mode
  int rows_cap;           // batch * (seqlen_q or max_seqlen_q): bound on query rows
  int ws_stride;          // rows_cap + kBwdPad
  int n_qtiles;           // dQ kernel: query tiles per (sequence, head), longest sequence
  int n_kblocks;          // dK/dV kernel: key blocks per (sequence, kv head), longest
  float scale;
  float c;                // scale * log2(e)
  int g_f32;              // gradients stored as fp32 (else bf16)
};

int bwd_dq_rows();       // query rows per dQ workgroup
int bwd_dkdv_keys();     // keys per dK/dV workgroup
hipError_t launch_bwd(const BwdParams& p, int head_dim, bool causal, hipStream_t stream);

// Which forward kernel a call runs, and its workgroup shape.
enum class FwdKind { Plain, Ext, Fp8 };
struct FwdPlan {
  int waves;       // waves per workgroup
  int block_rows;  // query rows per workgroup tile
  int wide;        // 64 query rows per wave
};
FwdPlan fwd_plan(FwdKind kind, int head_dim, bool causal, bool varlen, int seqlen_q);
hipError_t launch_fwd(const FwdParams& p, int head_dim, bool causal, hipStream_t stream);
// Head dim 128, plain attention: 64 query rows per wave (p.waves = 2 or 4).
hipError_t launch_fwd_wide(const FwdParams& p, bool causal, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int head_dim, hipStream_t stream);
// FP8 forward (head dim 128): p.c = scale * q_descale * k_descale * log2(e).
hipError_t launch_fwd_fp8(const FwdParams& p, bool causal, float v_descale, hipStream_t stream);
hipError_t launch_fwd_local(const FwdParams& p, int head_dim, bool causal, int win_left,
                            int win_right, hipStream_t stream);
hipError_t launch_fwd_xf(const FwdParams& p, int head_dim, bool causal, int win_left,
                         int win_right, float scale, float cap, const float* alibi,
                         int alibi_stride, hipStream_t stream);
hipError_t launch_append(const AppendParams& a, int head_dim, hipStream_t stream);
hipError_t launch_combine(const float* o_part, const float* lse_part, int rows, int n_splits,
                          int head_dim, void* o, float* lse, int o_f32, hipStream_t stream);

}  // namespace fa
