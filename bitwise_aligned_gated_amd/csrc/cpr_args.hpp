// cpr_args.hpp -- plain-C++ kernel argument blocks shared by the host library and the kernels.
#pragma once

#include <stdint.h>

namespace cpr {

struct PrefillArgs {
  const int32_t* cu;          // [num_seqs + 1]
  const int32_t* slot_ids;    // [num_seqs]
  const int64_t* pos;         // [num_slots] (read)
  int64_t* pos_out;           // same array, written only by the finish kernel
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  void* o;
  float* state;               // [num_slots][H_v][dv][dk]
  float* chunk_states;        // [rows_cap][H_v][dv][dk]
  int64_t total_tokens;
  int64_t rows_cap;
  int32_t num_seqs;
  int32_t num_slots;
  int32_t from_state;
  int32_t h_k;
  int32_t h_v;
  int32_t chunk;
  int32_t round_boundary;     // 1: bf16 boundary dtype (round the state at chunk starts)
  void* const* events;        // nullable: hipEvent_t recorded around the kernels
};

struct DecodeArgs {
  const int32_t* slot_ids;    // [batch]
  int64_t* pos;               // [num_slots]
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  void* o;
  float* state;
  float* boundary;            // nullable: [num_slots][H_v][dv][dk]
  int64_t* boundary_pos;      // nullable: [num_slots]
  int32_t batch;
  int32_t num_slots;
  int32_t h_k;
  int32_t h_v;
  int32_t chunk;
  int32_t round_boundary;     // 1: bf16 boundary dtype (round the state at chunk starts)
  void* const* events;        // nullable: 2 hipEvent_t recorded around the step kernel
};

}  // namespace cpr
