// Kernel parameter blocks (plain structs passed by value to the kernels).
#pragma once
#include <stdint.h>

namespace gqla {

struct DecodeParams {
  const uint16_t* q_nope;        // [B][s_q][h_q][d_nope]
  const uint16_t* q_rope;        // [B][s_q][h_q][d_rope]
  const uint16_t* cache;         // latent or expanded pages
  const int32_t* block_table;    // [B][max_blocks]
  const int32_t* seqlens;        // [B]
  const uint16_t* w_uk;          // [g][r][d_nope]   (absorb path only)
  const uint16_t* w_uv;          // [g][r][d_v]      (absorb path only)
  const int32_t* split_offsets;  // [B+1] or nullptr
  uint16_t* qcat;                // absorb path: [B][s_q][h_q][r + d_rope] workspace
  uint16_t* wuvT;                // absorb path: [g][d_v][r] workspace (W_UV transposed)
  uint16_t* olat;                // absorb path: [units][s_q][h_q][r] workspace (split o_lat, bf16)
  float* olse;                   // absorb path: [units][s_q][h_q] workspace (split lse)
  uint16_t* out;                 // [B][s_q][h_q][d_v] bf16 (unsplit launch)
  float* lse;                    // [B][s_q][h_q] or nullptr (unsplit launch)
  float* part_out;               // [S][s_q][h_q][d_v] (split launch)
  float* part_lse;               // [S][s_q][h_q]      (split launch)
  int32_t batch;
  int32_t max_blocks;
  int32_t num_groups;
  int32_t split_tokens;          // tokens per split (split launch)
  int32_t num_units;             // total splits, or batch when unsplit
  float scale_log2;              // softmax scale * log2(e)
  const uint32_t* codes;         // sparse GQA: row codes [B][g][topk_pad], else nullptr
  int32_t topk_pad;              // sparse GQA: entries per (sequence, group), a multiple of 32
};

struct SparseCodeParams {
  const int32_t* indices;        // [B][g][topk] token positions
  const int32_t* block_table;    // [B][max_blocks]
  const int32_t* seqlens;        // [B]
  uint32_t* codes;               // [B][g][topk_pad]
  int64_t num_pages;
  int32_t batch;
  int32_t num_groups;
  int32_t topk;
  int32_t topk_pad;
  int32_t max_blocks;
  int32_t block_size;
  int32_t s_q;
  int32_t* split_offsets;        // [B + 1] split plan (i * splits_per_seq), or nullptr
  int32_t splits_per_seq;
};

struct ExpandParams {
  const uint16_t* latent;        // [n_pages][bs][r + d_rope]
  const uint16_t* w_uk;          // [g][r][d_nope]
  const uint16_t* w_uv;          // [g][r][d_v]
  const int32_t* page_ids;       // [n] or nullptr
  uint16_t* expanded;            // [n_pages][page_elems]
  int64_t n_expand;              // pages to expand
  int32_t num_groups;
  // expand_pages_kernel: workgroups [0, whole_quads) take page quads whole,
  // the rest take one of `pieces` pass ranges of each following quad
  int64_t whole_quads;
  int32_t pieces;
};

struct AppendParams {
  const uint16_t* new_rows;      // [batch][n_new][row_elems]
  uint16_t* latent;              // [n_pages][bs][row_elems]
  const int32_t* block_table;    // [batch][max_blocks]
  const int32_t* seqlens;        // [batch], counting the new tokens
  const uint16_t* w_uk;          // [g][r][d_nope]  (with expanded)
  const uint16_t* w_uv;          // [g][r][d_v]     (with expanded)
  uint16_t* expanded;            // [n_pages][page_elems], or nullptr (latent only)
  int64_t row_elems;             // r + d_rope
  int32_t num_groups;
  int32_t batch;
  int32_t n_new;
  int32_t max_blocks;
  int32_t bs;
};

struct CombineParams {
  const float* part_out;         // [S][rows][d_v]
  const float* part_lse;         // [S][rows]
  const int32_t* split_offsets;  // [B+1]
  uint16_t* out;                 // [B][rows][d_v]
  float* lse;                    // [B][rows] or nullptr
  int32_t batch;
  int32_t rows;                  // s_q * h_q
};

}  // namespace gqla
