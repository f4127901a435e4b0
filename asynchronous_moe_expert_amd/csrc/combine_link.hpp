// The link step of the combine's list path for one arrival ([SEP] section 3: an arriving
// expert result is buffered against its token until all K have arrived): range and
// generation checks, then a push onto the token's arrival list (head[t] = newest arrival,
// next[i] = the one pushed before it), with the token's mask at that point kept in mpre[i].
// Used by the combine's link kernel and by the queue-index kernel, which links the arrivals of
// the FFN call it indexes as soon as their batch rows are known.  Self-contained (the error
// bits of moe_step.h; atomicOr, atomicExch, min and max from the including translation unit),
// so that the host build of the combine kernels can include it too.
#pragma once
#include <stdint.h>

#include "moe_step.h"

namespace moe {

struct LinkJob {
  int m = 0;  // arrivals (0: nothing to link)
  int K = 0, T_cap = 0;
  int64_t n_rows = 0;
  const int32_t* tok = nullptr;
  const int32_t* kslot = nullptr;
  const uint32_t* gen = nullptr;
  const uint32_t* tgen = nullptr;
  const uint32_t* mask = nullptr;
  int32_t* head = nullptr;
  int32_t* next = nullptr;   // [m] (workspace)
  uint32_t* mpre = nullptr;  // [m] (workspace)
  uint32_t* err = nullptr;
};

// an arrival's metadata, then its token's mask and generation (two dependent loads; the
// second is clamped into the state, and only used when the token is in range)
struct LinkIn {
  int t = 0, k = 0;
  uint32_t g = 0u, m_t = 0u, tg = 0u;
};

__device__ __forceinline__ LinkIn link_load_meta(const LinkJob& j, int i) {
  LinkIn a;
  a.t = j.tok[i];
  a.k = j.kslot[i];
  a.g = j.gen[i];
  return a;
}

__device__ __forceinline__ void link_load_state(const LinkJob& j, LinkIn& a) {
  const int tc = min(max(a.t, 0), j.T_cap - 1);
  a.m_t = j.mask[tc];  // (no kernel of this call has changed it yet)
  a.tg = j.tgen[tc];
}

// arrival i with batch row r (a row outside [0, n_rows) is an error)
__device__ __forceinline__ void link_push(const LinkJob& j, int i, int64_t r, const LinkIn& a) {
  unsigned flag = 0u;
  if (a.t < 0 || a.t >= j.T_cap) flag |= MOE_ERR_TOKEN_RANGE;
  if (a.k < 0 || a.k >= j.K) flag |= MOE_ERR_KSLOT_RANGE;
  if (r < 0 || r >= j.n_rows) flag |= MOE_ERR_ROW_RANGE;
  if (!flag && a.g != a.tg) flag |= MOE_ERR_STALE_GEN;
  if (flag) {
    atomicOr(j.err, flag);
    j.next[i] = -2;  // not linked
    return;
  }
  j.mpre[i] = a.m_t;
  j.next[i] = atomicExch(&j.head[a.t], i);
}

// Host side.  combine.hip: validates a combine call like moe_combine_plan; on MOE_OK *job is the
// call's link step when it takes the list path, job->m = 0 otherwise.  assemble.hip: whether
// the index of a queue of n pairs can link its arrivals, and moe_assemble with the arrivals'
// link step in the same launch (arrival i is queue entry i, its batch row pos[i]).
int combine_link_job(const moe_combine_args* a, LinkJob* job);
bool assemble_links(int n);
int assemble_with_link(const moe_assemble_args* a, const LinkJob& link, hipStream_t stream);

}  // namespace moe
