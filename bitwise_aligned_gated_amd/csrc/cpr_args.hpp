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
  float* c_stash;             // nullable: [N][H_v][dv] fp32, every token's c (pass 1 writes, pass 2 reads)
  float* w_stash;             // nullable (needs c_stash): [N][H_v][dv] fp32, every token's w
  void* const* events;        // nullable: hipEvent_t recorded around the kernels
  int64_t grid_items;         // set per launch: the kernel's work items (one per natural workgroup)
  int64_t max_wgs;            // 0: one workgroup per item; else at most this many, taking items in turn
  uint32_t* status;           // overlapped kernel: device word a bounded wait that gives up ORs a flag into
  uint32_t wait_limit;        // overlapped kernel: polls per bounded wait (0: the default)
  const int32_t* gate;        // chunk-form kernels, nullable: sequence j runs only where gate[j] != 0, and then
                              //   as one chunk row (row j) of C tokens (the decode resynchronisation)
  const float* state_in;      // chunk-form state pass, nullable: where continuing sequences start (else state)
  void* r2_ring;              // chunked R2 prefill, nullable: the pool's decode ring to fill
  float* r2_boundary;         //   and its boundary record (state and position) to set
  int64_t* r2_boundary_pos;
  float* chunk_bwd;           // chunk-form prep, nullable: T^T and W^T per (chunk row, value head) for the
                              //   chunk-form backward (the chunk-form state pass then also writes c_stash)
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
  int64_t grid_items;         // set per launch: the kernel's work items
  int64_t max_wgs;            // 0: one workgroup per item; else at most this many, taking items in turn
  int32_t skip_advance;       // 1: leave the positions to a later kernel (the R2 ring append)
  const int32_t* skip_slot;   // nullable [num_slots]: a slot with skip_slot[slot] != 0 is stepped by a later
                              //   launch (R2: the slots the chunk form resynchronises, on a second stream)
};

// Gradients of a forward that started every sequence at position 0 (the trainer's case).
struct BackwardArgs {
  const int32_t* cu;          // [num_seqs + 1]
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  const void* d_o;            // [N][H_v][dv], io dtype
  const float* d_state;       // nullable: [num_seqs][H_v][dv][dk] gradient of the final states
  const float* chunk_states;  // the forward's stash: [rows][H_v][dv][dk]
  float* adjoint;             // workspace [adj_rows][H_v][dv][dk]: dL/dS at every chunk boundary
  float* dc;                  // workspace [N][H_v][dv]: (G_t + q_t dO_t^T)^T k_t
  float* cc;                  // workspace [N][H_v][dv]: c_t of the forward
  float* ww;                  // workspace [N][H_v][dv]: w_t of the forward
  double* hpart;              // workspace [adj_rows][H_v][partials]: <G, S> at each chunk start, in parts
  float* xv;                  // workspace [N][H_v]: v_t . dv_t
  float* dq;                  // [N][H_k][dk]
  float* dk;                  // [N][H_k][dk]
  float* dv;                  // [N][H_v][dv]
  float* da;                  // [N][H_v]
  float* db;                  // [N][H_v]
  float* d_state0;            // nullable: [num_seqs][H_v][dv][dk]
  int64_t total_tokens;
  int64_t rows_cap;           // chunk rows any plan can use
  int64_t adj_rows;           // rows_cap + num_seqs (each sequence has one boundary more than chunks)
  int32_t num_seqs;
  int32_t h_k;
  int32_t h_v;
  int32_t chunk;
  int32_t have_cw;            // 1: cc and ww came from the trainer forward (no replay needed)
  int32_t hparts;             // parts of <G, S> per chunk start and value head in hpart
  void* const* events;        // nullable: 4 hipEvent_t around the three kernels
  const float* fws;           // chunk-form backward: the forward's per-chunk workspace (W, U, C^T, log gates)
  const float* fbw;           //   and what its prep kept for the backward (T^T, W^T)
};

}  // namespace cpr
