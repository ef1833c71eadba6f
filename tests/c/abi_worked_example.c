/* Plain C11 caller of the C ABI: plans the EPIC walkthrough's worked example (chunks of
 * 4, 5 and 5 tokens, 3 query tokens, k = 2) with pic_build_index and prints the plan's
 * recompute positions and offsets, one line each.  Host only: no device call. */
#include <stdio.h>
#include <stdlib.h>

#include "pic.h"

int main(void) {
  const int32_t req_chunk_ptr[2] = {0, 3};
  const int32_t chunk_lens[3] = {4, 5, 5};
  const int32_t q_lens[1] = {3};
  int64_t words = 0;
  int st = pic_build_index(1, req_chunk_ptr, chunk_lens, q_lens, NULL, 2, 0, 4, 4, 0, NULL, 0,
                           &words);
  if (st != PIC_ENOSPC && st != PIC_OK) {
    fprintf(stderr, "size query: %s\n", pic_strerror(st));
    return 1;
  }
  int32_t *plan = (int32_t *)calloc((size_t)words, sizeof(int32_t));
  if (!plan) return 1;
  st = pic_build_index(1, req_chunk_ptr, chunk_lens, q_lens, NULL, 2, 0, 4, 4, 0, plan, words,
                       &words);
  if (st != PIC_OK) {
    fprintf(stderr, "plan: %s\n", pic_strerror(st));
    return 1;
  }
  const int32_t *rows = plan + plan[PIC_H_O_ROWS];
  printf("rows");
  for (int32_t r = 0; r < plan[PIC_H_N_ROWS]; ++r) printf(" %d", rows[r]);
  printf("\noffsets");
  const int32_t *off = plan + plan[PIC_H_O_CHUNK_OFF];
  for (int32_t c = 0; c <= plan[PIC_H_N_CHUNKS]; ++c) printf(" %d", off[c]);
  printf("\ntokens %d\n", plan[PIC_H_N_TOKENS]);
  printf("bad plan: %s\n", pic_strerror(pic_build_index(-1, req_chunk_ptr, chunk_lens, q_lens,
                                                        NULL, 2, 0, 4, 4, 0, NULL, 0, &words)));
  free(plan);
  return 0;
}
