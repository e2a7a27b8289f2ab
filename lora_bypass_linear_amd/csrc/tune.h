// tune.h -- the measured tile pick's table (internal to the library).
#pragma once

#include <stdint.h>

#include <string>

namespace lyc {

struct TuneChoice {
    int tile, ksplit;
    double ms;
};

// Key of a LoRA forward on the current device: device | op | M bucketed to a
// power of two | N | K | padded rank | compute | output dtype.  Empty when no
// device is current.
std::string tune_key(const char* op, int64_t M, int64_t N, int64_t K, int r_pad, int c_dt, int o_dt);
bool tune_lookup(const std::string& key, TuneChoice* out);
void tune_store(const std::string& key, const TuneChoice& c);
int tune_count();
void tune_clear();
// JSON table; 0 on success
int tune_save(const char* path);
int tune_load(const char* path, int* loaded);

}  // namespace lyc
