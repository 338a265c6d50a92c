// Internal declarations of the sparse attention over the selected keys (the consumer of the
// indexer's top-k).  The exported C ABI is include/dsa_indexer.h; nothing here crosses it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kLatentDim = 512;     // main-KV latent: key and value of every head
constexpr int kAttnChunk = 32;      // listed keys staged per step
constexpr int kMaxAttnList = 2048;  // list entries one workgroup resolves (1024 with 32 heads)

// List entries one workgroup resolves for n_heads heads: eight per thread.
constexpr int attn_max_list(int n_heads) { return n_heads == 32 ? kMaxAttnList / 2 : kMaxAttnList; }

struct AttnArgs {
  const uint16_t* q;        // [n_q, H, 512] bf16
  const uint16_t* kv;       // [n_slots, 512] bf16
  int64_t n_slots;
  const int32_t* kv_slot;   // [n_seq, max_keys]: kv row of key s of sequence b
  int32_t n_seq;
  int32_t max_keys;
  const int32_t* cu_q;      // [n_seq + 1]
  const int32_t* idx;       // [n_q, k] listed key indices, -1 = none
  int64_t n_q;
  int32_t n_heads;          // 32, 64 or 128
  int32_t k;
  float scale_log2;         // softmax scale times log2(e)
  int32_t n_split;          // workgroups per query row, each over split_keys list entries
  int32_t split_keys;       // a multiple of kAttnChunk
  uint16_t* out;            // [n_q, H, 512] bf16, written when n_split == 1 and by the merge
  float* lse;               // [n_q, H] natural-log log-sum-exp, or null
  float* part_o;            // [n_q, n_split, H, 512] unnormalised partial outputs (n_split > 1)
  float* part_ml;           // [n_q, n_split, H, 2] partial (max in log2 units, weight sum)
};

// Splits per query row and entries per split for a batch; workspace bytes for the partials.
void attn_plan(int64_t n_q, int32_t n_heads, int32_t k, int32_t* n_split, int32_t* split_keys);
size_t attn_workspace_bytes(int64_t n_q, int32_t n_heads, int32_t k);

hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace dsa
