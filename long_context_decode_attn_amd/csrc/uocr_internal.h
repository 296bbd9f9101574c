// Internal interface between the C-ABI layer (uocr_api.cpp) and the gfx950
// kernels (uocr_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace uocr {

struct AppendArgs {
  void* k_ring;
  void* v_ring;
  const void* k_new;
  const void* v_new;
  int32_t* t_gen;
  int batch, heads, window;
};

struct DecodeArgs {
  const void* q;
  const void* k_prefix;
  const void* v_prefix;
  const int32_t* prefix_len;
  const void* k_ring;
  const void* v_ring;
  const int32_t* t_gen;
  void* out;
  float* part_ml;      // splits > 1: [units][splits][2] (max, sum)
  float* part_o;       // splits > 1: [units][splits][D]
  int units, heads, prefix_cap, window;
  int splits;          // workgroups per unit (partials merged by k_split_merge when > 1)
  int chunk;           // dense: keys per split
  int waves;           // waves per workgroup
  float qscale;        // scale * log2(e)
  // sparse only
  const int32_t* sel_idx;
  const float* sel_bias;
  int topk;
};

struct IndexArgs {
  const void* k_prefix;
  const int32_t* prefix_len;
  const float* proj;
  float* kbar;
  int units, heads, prefix_cap, nb_cap;
  int first_block, n_blocks;  // blocks [first_block, first_block + n_blocks) of every unit
};

struct ScoreArgs {
  const void* q;
  const float* proj;
  const float* kbar;
  const int32_t* prefix_len;
  float* scores;
  int units, heads, prefix_cap, nb_cap;
  int parts;           // workgroups per unit
};

struct TopkArgs {
  const float* scores;
  const int32_t* prefix_len;
  int32_t* sel_idx;
  float* sel_prob;
  float* sel_bias;
  int units, heads, prefix_cap, nb_cap, topk;
};

// Prefill-side routing of a chunk of tq queries per unit.
struct PrefillArgs {
  const void* q;          // [units][tq][D]
  const int32_t* q_pos;   // [batch] position of query 0 of the chunk
  const float* proj;      // [D][32]
  const float* kbar;      // [units][nb_cap][32]
  const int32_t* prefix_len;
  int32_t* sel_idx;       // [units][tq][topk]
  float* sel_prob;        // may be null
  float* sel_bias;
  int units, heads, prefix_cap, nb_cap, topk, tq, qt;
};

// Windowed no-repeat n-gram ban and page guard over one step's logits.
struct NgramArgs {
  const int32_t* tokens;      // [batch][ring_cap] generated token pos at pos % ring_cap
  const int32_t* n_gen;       // [batch]
  const int32_t* page_tokens; // [batch] tokens of the current page (may be null: no guard)
  void* logits;               // [batch][vocab]
  int batch, ring_cap, ngram, window, page_token, eos_token, max_page_tokens, vocab;
};
constexpr int kMaxNgramWindow = 4096;

// page2d rotary embedding of x and (if not null) y, both [batch][heads][tokens][D],
// in place, with the positions of token t of sequence b at page[b * tokens + t],
// offset[...].
constexpr int kRopeTokens = 16;  // tokens of one sequence per workgroup
struct RopeArgs {
  void* x;
  void* y;
  const int32_t* page;
  const int32_t* offset;
  int batch, heads, tokens, page_mod;
  float base;
};

// A fused decode step: DecodeArgs plus the new token, the double-buffered
// generated-token counts and (SR-SWA) the routing inputs and outputs.
struct StepArgs {
  DecodeArgs d;        // d.k_ring / d.v_ring alias k_ring / v_ring below
  const void* k_new;
  const void* v_new;
  void* k_ring;
  void* v_ring;
  const int32_t* t_gen_in;
  int32_t* t_gen_out;
  const float* proj;
  const float* kbar;
  int nb_cap;
  int32_t* sel_idx;
  float* sel_prob;
  float* sel_bias;
  // page2d rotation of q and k_new before use (rope_page == null: none):
  // the new token of sequence b sits at (rope_page[b], rope_offset[b])
  const int32_t* rope_page;
  const int32_t* rope_offset;
  int rope_page_mod;
  float rope_base;
};

constexpr int kBlock = 32;     // tokens per routing block
constexpr int kIdxDim = 32;    // index projection width
constexpr int kMaxBlocks = 4096;
constexpr int kMaxTopk = 64;

hipError_t launch_ring_append(int dtype, int head_dim, const AppendArgs& a, hipStream_t s);
hipError_t launch_rswa_decode(int dtype, int head_dim, const DecodeArgs& a, hipStream_t s);
hipError_t launch_srswa_decode(int dtype, int head_dim, const DecodeArgs& a, hipStream_t s);
hipError_t launch_block_index(int dtype, int head_dim, const IndexArgs& a, hipStream_t s);
hipError_t launch_block_score(int dtype, int head_dim, const ScoreArgs& a, hipStream_t s);
hipError_t launch_entmax_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_prefill_route(int dtype, int head_dim, const PrefillArgs& a, hipStream_t s);
int prefill_queries_per_wg(int nb_cap);
hipError_t launch_ngram_ban(int dtype, const NgramArgs& a, hipStream_t s);
hipError_t launch_rope_page2d(int dtype, int head_dim, const RopeArgs& a, hipStream_t s);
hipError_t launch_srswa_step(int dtype, int head_dim, const StepArgs& a, hipStream_t s);
hipError_t launch_rswa_step(int dtype, int head_dim, const StepArgs& a, hipStream_t s);

// Phase stamps of the last fused SR-SWA steps (a library built with
// UOCR_PHASE_STAMPS; hipErrorNotSupported otherwise): copies the first
// `bytes` of the [kMaxStampUnits][64] uint64 stamp array to host memory and
// waits for the copy.
constexpr int kMaxStampUnits = 4096;
hipError_t read_phase_stamps(void* dst, size_t bytes, hipStream_t s);

}  // namespace uocr
