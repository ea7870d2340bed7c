"""Inner-product search over TurboQuant codes (fp64).

[TurboQuant-es] "Velocidad y eficiencia de indexación" and [TurboQuant-pl]
"Zaskakujące przyspieszenie baz wektorowych": nearest-neighbour search by
inner product over vectors encoded with the data-oblivious codec, so that
indexing is only the encode.  The score of a database row is the unbiased
code-domain estimate; the top-k list is sorted by descending estimate with
ties going to the lower database index.
"""

import numpy as np

from .codec import estimate_ip


def inner_product_matrix(q, codes, book):
    """(n_q, n) estimates of <q_a, x_j>; codes: dict idx, norm[, sign,
    rnorm]; book: dict signs, centroids[, S]."""
    return estimate_ip(q, codes["idx"], codes["norm"], book["signs"], book["centroids"],
                       sign=codes.get("sign"), rnorm=codes.get("rnorm"), S=book.get("S"))


def top_k(scores, k):
    """Indices and values of the k largest scores per row, descending, ties
    to the lower index (a stable sort of the negated scores)."""
    scores = np.asarray(scores, dtype=np.float64)
    order = np.argsort(-scores, axis=1, kind="stable")[:, :k]
    return order, np.take_along_axis(scores, order, axis=1)
